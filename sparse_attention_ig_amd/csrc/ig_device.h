// Device helpers for the gfx950 kernels: element loads, bf16 widening,
// wavefront (64-lane) reductions and the order-preserving score key.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ig {

constexpr int kWave = 64;

// Elements per 16-byte load.
template <typename T> struct Vec;
template <> struct Vec<float> { static constexpr int N = 4; };
template <> struct Vec<uint16_t> { static constexpr int N = 8; };

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// 16-byte load of N elements, widened to float.
__device__ __forceinline__ void load_vec(const float* __restrict__ p, float (&v)[4]) {
    float4 t = *reinterpret_cast<const float4*>(p);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
}
__device__ __forceinline__ void load_vec(const uint16_t* __restrict__ p, float (&v)[8]) {
    uint4 t = *reinterpret_cast<const uint4*>(p);
    v[0] = __uint_as_float(t.x << 16); v[1] = __uint_as_float(t.x & 0xFFFF0000u);
    v[2] = __uint_as_float(t.y << 16); v[3] = __uint_as_float(t.y & 0xFFFF0000u);
    v[4] = __uint_as_float(t.z << 16); v[5] = __uint_as_float(t.z & 0xFFFF0000u);
    v[6] = __uint_as_float(t.w << 16); v[7] = __uint_as_float(t.w & 0xFFFF0000u);
}

// Widen a raw 16-byte word to floats (8 bf16 or 4 f32).
__device__ __forceinline__ void unpack_raw(const uint4& t, float (&v)[8]) {
    v[0] = __uint_as_float(t.x << 16); v[1] = __uint_as_float(t.x & 0xFFFF0000u);
    v[2] = __uint_as_float(t.y << 16); v[3] = __uint_as_float(t.y & 0xFFFF0000u);
    v[4] = __uint_as_float(t.z << 16); v[5] = __uint_as_float(t.z & 0xFFFF0000u);
    v[6] = __uint_as_float(t.w << 16); v[7] = __uint_as_float(t.w & 0xFFFF0000u);
}
__device__ __forceinline__ void unpack_raw(const uint4& t, float (&v)[4]) {
    v[0] = __uint_as_float(t.x); v[1] = __uint_as_float(t.y);
    v[2] = __uint_as_float(t.z); v[3] = __uint_as_float(t.w);
}

// Raw 16-byte copy helpers (no widening).
__device__ __forceinline__ uint4 load_raw16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void store_raw16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return bf16_to_f32(v); }

// Sum over groups of G consecutive lanes (G a power of two <= 64); every lane of
// the group gets the group total.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int m = 1; m < G; m <<= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
    return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
        uint32_t o = __shfl_xor(v, m, kWave);
        v = o > v ? o : v;
    }
    return v;
}
__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

// Order-preserving map float -> uint32 (larger float -> larger key); -0 maps
// like +0 so that equal scores give equal keys.
__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

// q[c] = sum over splits of part[s][b][col0 + c] (+ bias[col0 + c]) for c < R, in split order.
// Every (split, c) load is issued by its own thread at once (a loop of dependent loads would cost
// one memory round trip per split); s_part holds NT floats.  Ends with a barrier; q (and q_out,
// when not NULL) then hold the sums.
template <int NT>
__device__ __forceinline__ void sum_partials(const float* __restrict__ part, int splits, int B, int N, int b,
                                             int col0, int R, const float* __restrict__ bias, float* q,
                                             float* s_part, float* q_out) {
    const int tid = threadIdx.x;
    const int per = NT / R;  // splits loaded per pass
    float a = 0.f;
    for (int s0 = 0; s0 < splits; s0 += per) {
        const int s = s0 + tid / R, c = tid % R;
        float v = 0.f;
        if (tid < per * R && s < splits) v = part[(static_cast<size_t>(s) * B + b) * N + col0 + c];
        s_part[tid] = v;
        __syncthreads();
        if (tid < R) {
            for (int k = 0; k < per && s0 + k < splits; ++k) a += s_part[k * R + tid];
        }
        __syncthreads();
    }
    if (tid < R) {
        if (bias) a += bias[col0 + tid];
        q[tid] = a;
        if (q_out) q_out[tid] = a;
    }
    __syncthreads();
}

// Lanes below this one in the wave, as a 64-bit mask.
__device__ __forceinline__ uint64_t lanemask_lt() {
    uint32_t lane = __lane_id();
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace ig
