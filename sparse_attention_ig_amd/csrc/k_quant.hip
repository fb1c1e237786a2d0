// INT4 KV pool records (InfiniGen, arXiv 2406.19707, paper-graph-ui summary:
// section 5 "Evaluation Methodology" names 4-bit group-wise asymmetric KV
// quantisation as a baseline, and the "Follow-Up Research" paragraph on
// combining prefetching with KV cache quantisation proposes storing the pool
// at that precision and fetching only the speculated rows).
//
// Record of one token's key and value rows of d elements each (d a multiple
// of 32), int4_record_bytes(d) bytes (160 for d = 128): K codes in bytes
// [0, d/2) and V codes in [d/2, d) (element i in byte i/2 of its half, low
// nibble for even i), then per group g of 32 elements, K groups first, a
// float16 step and a float16 minimum (bytes d + 4g .. +4), then zero padding
// to a multiple of 32 bytes.  One record per token keeps a fetched row to
// three 64-byte host-link requests (eight for a bf16 K and V row), which is
// what bounds a scattered gather over the link.
// Per group: mn, mx over its 32 values; s16 = half((mx - mn) / 15), m16 =
// half(mn) (nearest-even); code = clamp(rint((v - m16) / s16), 0, 15), 0 when
// s16 is 0 (float32, correctly rounded division, round half to even).
//
//   k_quant          one thread per group: rows [row0, row0 + nrows) of bf16 /
//                    f32 K and V caches to records (destination row = source
//                    row, or slot[b] + row - row0 for an append)
//   k_gather_q4      one thread per group of a selected record (device or
//                    host-mapped memory): dequantised, v = m16 + code * s16 in
//                    float32, into compact K and V rows
#include <algorithm>
#include <hip/hip_fp16.h>

#include "ig_device.h"
#include "ig_internal.h"

namespace ig {

constexpr int kQGroup = 32;
constexpr int kQThreads = 256;

size_t int4_record_bytes(int d) { return (static_cast<size_t>(d) + static_cast<size_t>(d) / 4 + 31) / 32 * 32; }

__device__ __forceinline__ void load_group(const uint16_t* p, float (&v)[kQGroup]) {
#pragma unroll
    for (int u = 0; u < kQGroup / 8; ++u) {
        float t[8];
        unpack_raw(load_raw16(p + 8 * u), t);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[8 * u + e] = t[e];
    }
}
__device__ __forceinline__ void load_group(const float* p, float (&v)[kQGroup]) {
#pragma unroll
    for (int u = 0; u < kQGroup / 4; ++u) {
        float t[4];
        unpack_raw(load_raw16(p + 4 * u), t);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * u + e] = t[e];
    }
}

template <typename T>
__global__ __launch_bounds__(kQThreads) void k_quant(const T* __restrict__ K, const T* __restrict__ V, int H, int d,
                                                     int ld_rows, int row0, int nrows, const int32_t* __restrict__ slot,
                                                     unsigned char* __restrict__ Xq, int q_rows, int rec,
                                                     int64_t total) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kQThreads + threadIdx.x;
    if (t >= total) return;
    const int gpr = d / kQGroup;
    const int g = static_cast<int>(t % (2 * gpr));  // K groups, then V groups
    const int64_t row = t / (2 * gpr);              // (bh, j) with j < nrows
    const int j = static_cast<int>(row % nrows);
    const int bh = static_cast<int>(row / nrows);
    const T* X = g < gpr ? K : V;
    float v[kQGroup];
    load_group(X + (static_cast<size_t>(bh) * ld_rows + row0 + j) * d + (g % gpr) * kQGroup, v);
    float mn = v[0], mx = v[0];
#pragma unroll
    for (int e = 1; e < kQGroup; ++e) {
        mn = fminf(mn, v[e]);
        mx = fmaxf(mx, v[e]);
    }
    const __half s16 = __float2half_rn((mx - mn) / 15.0f);
    const __half m16 = __float2half_rn(mn);
    const float sf = __half2float(s16), mf = __half2float(m16);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < kQGroup; ++e) {
        int q = 0;
        if (sf > 0.f) q = min(max(static_cast<int>(rintf((v[e] - mf) / sf)), 0), 15);
        w[e / 8] |= static_cast<uint32_t>(q) << (4 * (e % 8));
    }
    int dj = slot ? slot[bh / H] + j : row0 + j;
    dj = min(max(dj, 0), q_rows - 1);
    unsigned char* r = Xq + (static_cast<size_t>(bh) * q_rows + dj) * rec;
    store_raw16(r + g * 16, make_uint4(w[0], w[1], w[2], w[3]));
    const uint32_t sm = static_cast<uint32_t>(__half_as_ushort(s16)) | (static_cast<uint32_t>(__half_as_ushort(m16)) << 16);
    *reinterpret_cast<uint32_t*>(r + d + g * 4) = sm;
    if (g == 0) {
        for (int pb = d + 8 * gpr; pb < rec; pb += 4) *reinterpret_cast<uint32_t*>(r + pb) = 0u;
    }
}

__device__ __forceinline__ void store_group(uint16_t* p, const float (&v)[kQGroup]) {
#pragma unroll
    for (int u = 0; u < kQGroup / 8; ++u) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w[e] = static_cast<uint32_t>(f32_to_bf16(v[8 * u + 2 * e])) |
                   (static_cast<uint32_t>(f32_to_bf16(v[8 * u + 2 * e + 1])) << 16);
        store_raw16(p + 8 * u, make_uint4(w[0], w[1], w[2], w[3]));
    }
}
__device__ __forceinline__ void store_group(float* p, const float (&v)[kQGroup]) {
#pragma unroll
    for (int u = 0; u < kQGroup / 4; ++u)
        store_raw16(p + 4 * u, make_uint4(__float_as_uint(v[4 * u]), __float_as_uint(v[4 * u + 1]),
                                          __float_as_uint(v[4 * u + 2]), __float_as_uint(v[4 * u + 3])));
}

__device__ __forceinline__ void dequant_group(const unsigned char* r, int d, int g, float (&v)[kQGroup]) {
    const uint4 c = load_raw16(r + g * 16);
    const uint32_t sm = *reinterpret_cast<const uint32_t*>(r + d + g * 4);
    const float sf = __half2float(__ushort_as_half(static_cast<unsigned short>(sm & 0xFFFFu)));
    const float mf = __half2float(__ushort_as_half(static_cast<unsigned short>(sm >> 16)));
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int e = 0; e < kQGroup; ++e)
        v[e] = mf + static_cast<float>((w[e / 8] >> (4 * (e % 8))) & 15u) * sf;
}

// One thread per group of a selected row.  As in the row gather, the work is cut into units of
// kGatherQ4Rows rows of one (b, h) that the workgroups walk, at most kGatherQ4HostWgs of them when the
// records are in host memory (so that the host-link reads leave most of the GPU to kernels on other
// streams), one per unit otherwise; each thread has two rows' records in flight.
constexpr int kGatherQ4Rows = 64;
constexpr int kGatherQ4HostWgs = 128;
template <typename TO>
__global__ __launch_bounds__(kQThreads) void k_gather_q4(const unsigned char* __restrict__ KVq,
                                                         const int32_t* __restrict__ idx,
                                                         const int32_t* __restrict__ count, int d, int q_rows,
                                                         int max_out, int rec, int chunks, int64_t units,
                                                         TO* __restrict__ Kc, TO* __restrict__ Vc) {
    const int gpr = d / kQGroup;
    const int rows_per_step = kQThreads / (2 * gpr);
    const int g = threadIdx.x % (2 * gpr), ri = threadIdx.x / (2 * gpr);  // K groups, then V groups
    if (ri >= rows_per_step) return;
    TO* dst_base = g < gpr ? Kc : Vc;
    for (int64_t u0 = blockIdx.x; u0 < units; u0 += gridDim.x) {
        const int64_t bh = u0 / chunks;
        const int i0 = static_cast<int>(u0 - bh * chunks) * kGatherQ4Rows;
        const int c = min(count[bh], max_out);
        const int i1 = min(c, i0 + kGatherQ4Rows);
        for (int i = i0 + ri; i < i1; i += 2 * rows_per_step) {
            const int ib = i + rows_per_step;
            const bool two = ib < i1;
            int j0 = idx[static_cast<size_t>(bh) * max_out + i];
            int j1 = two ? idx[static_cast<size_t>(bh) * max_out + ib] : 0;
            j0 = min(max(j0, 0), q_rows - 1);
            j1 = min(max(j1, 0), q_rows - 1);
            float v0[kQGroup], v1[kQGroup];
            dequant_group(KVq + (static_cast<size_t>(bh) * q_rows + j0) * rec, d, g, v0);
            if (two) dequant_group(KVq + (static_cast<size_t>(bh) * q_rows + j1) * rec, d, g, v1);
            store_group(dst_base + (static_cast<size_t>(bh) * max_out + i) * d + (g % gpr) * kQGroup, v0);
            if (two) store_group(dst_base + (static_cast<size_t>(bh) * max_out + ib) * d + (g % gpr) * kQGroup, v1);
        }
    }
}

int launch_quantize(const void* K, const void* V, int B, int H, int d, int ld_rows, int dtype, int row0, int nrows,
                    const int32_t* slot, void* Xq, int q_rows, hipStream_t s) {
    const int64_t total = static_cast<int64_t>(B) * H * nrows * 2 * (d / kQGroup);
    if (total == 0) return 0;
    const dim3 grid(static_cast<unsigned>((total + kQThreads - 1) / kQThreads));
    const int rec = static_cast<int>(int4_record_bytes(d));
    if (dtype == IG_BF16)
        hipLaunchKernelGGL((k_quant<uint16_t>), grid, dim3(kQThreads), 0, s, static_cast<const uint16_t*>(K),
                           static_cast<const uint16_t*>(V), H, d, ld_rows, row0, nrows, slot,
                           static_cast<unsigned char*>(Xq), q_rows, rec, total);
    else
        hipLaunchKernelGGL((k_quant<float>), grid, dim3(kQThreads), 0, s, static_cast<const float*>(K),
                           static_cast<const float*>(V), H, d, ld_rows, row0, nrows, slot,
                           static_cast<unsigned char*>(Xq), q_rows, rec, total);
    return static_cast<int>(hipGetLastError());
}

int launch_gather_q4(const void* KVq, const int32_t* idx, const int32_t* count, int B, int H, int d, int q_rows,
                     int max_out, int dtype_out, void* Kc, void* Vc, hipStream_t s) {
    const int chunks = (max_out + kGatherQ4Rows - 1) / kGatherQ4Rows;
    const int64_t units = static_cast<int64_t>(chunks) * B * H;
    const dim3 grid(static_cast<unsigned>(std::min<int64_t>(units, host_resident(KVq) ? kGatherQ4HostWgs : (1 << 30))));
    const int rec = static_cast<int>(int4_record_bytes(d));
    const auto* kv = static_cast<const unsigned char*>(KVq);
    if (dtype_out == IG_BF16)
        hipLaunchKernelGGL((k_gather_q4<uint16_t>), grid, dim3(kQThreads), 0, s, kv, idx, count, d, q_rows, max_out,
                           rec, chunks, units, static_cast<uint16_t*>(Kc), static_cast<uint16_t*>(Vc));
    else
        hipLaunchKernelGGL((k_gather_q4<float>), grid, dim3(kQThreads), 0, s, kv, idx, count, d, q_rows, max_out,
                           rec, chunks, units, static_cast<float*>(Kc), static_cast<float*>(Vc));
    return static_cast<int>(hipGetLastError());
}

}  // namespace ig
