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
// float32 -> bfloat16 bits, round to nearest even (NaN stays a quiet NaN)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

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

// Cross-lane moves through DPP (data-parallel primitives: a VALU operand modifier, no LDS round
// trip).  GFX9 control codes: quad permutations, shifts within a 16-lane row, mirrors, and the row
// broadcasts used by wave scans.  Lanes without a source (or in rows left out by row_mask) read 0.
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRowMirror = 0x140;  // lane i <- lane 15 - i of its row
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7 - i of its half row
constexpr int kDppRowShr = 0x110;     // + k: lane i <- lane i - k of its row
constexpr int kDppBcast15 = 0x142;    // row r <- lane 15 of row r - 1
constexpr int kDppBcast31 = 0x143;    // rows 2, 3 <- lane 31

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i32(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(dpp_i32<CTRL>(__float_as_int(v)));
}

// Sum over groups of G consecutive lanes (G a power of two <= 64); every lane of the group gets the
// group total, the same value in every lane (each step adds two partial sums that the partner lane
// adds in the other order).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "group of 1, 2, 4, .., 64 lanes");
    if constexpr (G >= 2) v += dpp_f32<kDppQuadXor1>(v);
    if constexpr (G >= 4) v += dpp_f32<kDppQuadXor2>(v);
    if constexpr (G >= 8) v += dpp_f32<kDppHalfMirror>(v);   // the other quad of the half row
    if constexpr (G >= 16) v += dpp_f32<kDppRowMirror>(v);   // the other half of the row
    if constexpr (G >= 32) v += __shfl_xor(v, 16, kWave);
    if constexpr (G >= 64) v += __shfl_xor(v, 32, kWave);
    return v;
}

// Inclusive prefix sum over the 64 lanes (lane i gets v_0 + .. + v_i): scans within each 16-lane row
// by shifts of 1, 2, 4, 8, then the row totals are carried into the rows above by two broadcasts.
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += dpp_i32<kDppRowShr + 1>(v);
    v += dpp_i32<kDppRowShr + 2>(v);
    v += dpp_i32<kDppRowShr + 4>(v);
    v += dpp_i32<kDppRowShr + 8>(v);
    v += dpp_i32<kDppBcast15, 0xA>(v);
    v += dpp_i32<kDppBcast31, 0xC>(v);
    return v;
}

__device__ __forceinline__ int read_lane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

// Wave-wide reductions with a wave-uniform result: DPP within each 16-lane row, then the four row
// results read into scalar registers.
__device__ __forceinline__ int wave_sum_i32(int v) {
    v += dpp_i32<kDppQuadXor1>(v);
    v += dpp_i32<kDppQuadXor2>(v);
    v += dpp_i32<kDppHalfMirror>(v);
    v += dpp_i32<kDppRowMirror>(v);
    return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) + __builtin_amdgcn_readlane(v, 32) +
           __builtin_amdgcn_readlane(v, 48);
}
__device__ __forceinline__ uint32_t max_u32(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max_u32(v, static_cast<uint32_t>(dpp_i32<kDppQuadXor1>(static_cast<int>(v))));
    v = max_u32(v, static_cast<uint32_t>(dpp_i32<kDppQuadXor2>(static_cast<int>(v))));
    v = max_u32(v, static_cast<uint32_t>(dpp_i32<kDppHalfMirror>(static_cast<int>(v))));
    v = max_u32(v, static_cast<uint32_t>(dpp_i32<kDppRowMirror>(static_cast<int>(v))));
    const int vi = static_cast<int>(v);
    return max_u32(max_u32(static_cast<uint32_t>(__builtin_amdgcn_readlane(vi, 0)),
                           static_cast<uint32_t>(__builtin_amdgcn_readlane(vi, 16))),
                   max_u32(static_cast<uint32_t>(__builtin_amdgcn_readlane(vi, 32)),
                           static_cast<uint32_t>(__builtin_amdgcn_readlane(vi, 48))));
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

// ------------------------------------------------------------------ matrix-core projection step
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// One 16x16 MFMA step per element type.  Operand lane layout (16x16xK): lane l supplies row l % 16
// of A (here x: one batch row) and column l % 16 of B (one partial-weight column), each with E
// consecutive k values of k-group l / 16; the 16x16 float result puts rows 4 (l / 16) .. + 3 of
// column l % 16 in lane l.  Only the pairing of A's and B's k values matters for the sum, and both
// operands use the same one.
template <typename T> struct ProjMma;
template <> struct ProjMma<uint16_t> {
    static constexpr int K = 32, E = 8, CHUNK = 8;  // k per step, elements per lane, steps in flight
    using vec = uint4;
    static __device__ __forceinline__ vec load(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
    static __device__ __forceinline__ vec zero() { return make_uint4(0, 0, 0, 0); }
    static __device__ __forceinline__ f32x4_t mma(vec a, vec b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
};
template <> struct ProjMma<float> {
    static constexpr int K = 4, E = 1, CHUNK = 16;
    using vec = float;
    static __device__ __forceinline__ vec load(const float* p) { return *p; }
    static __device__ __forceinline__ vec zero() { return 0.f; }
    static __device__ __forceinline__ f32x4_t mma(vec a, vec b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

}  // namespace ig
