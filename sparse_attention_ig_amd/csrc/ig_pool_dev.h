// Block-level pool finish for one sequence (InfiniGen, arXiv 2406.19707,
// paper-graph-ui summary, section 3.4 "KV Cache Pool Management Under Memory
// Pressure"): clamp-and-halve every counter when one saturated, then the
// victim = lowest index among the minima.  Shared by the standalone touch
// kernel and the fused speculation kernel.
#pragma once

#include "ig_device.h"

namespace ig {

__device__ __forceinline__ uint32_t coherent_load(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// row: the n counters of one sequence.  All threads of the block call this;
// each thread touches only the slots j = tid (mod blockDim.x), so no barrier is
// needed between the halving and the argmin.  Returns the victim in thread 0.
template <int NT>
__device__ int pool_finish(uint32_t* __restrict__ row, int n, uint32_t cmax, bool halve, bool want_victim,
                           uint32_t* s_val, int* s_idx) {
    const int tid = threadIdx.x;
    constexpr int U = 8;  // 8 loads per lane in flight at a time
    if (halve) {
        for (int j0 = tid; j0 < n; j0 += NT * U) {
            uint32_t v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = j0 + u * NT < n ? coherent_load(&row[j0 + u * NT]) : 0u;
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (j0 + u * NT < n) row[j0 + u * NT] = (v[u] < cmax ? v[u] : cmax) >> 1;
        }
    }
    if (!want_victim) return -1;
    uint32_t best = 0xFFFFFFFFu;
    int bi = n;
    for (int j0 = tid; j0 < n; j0 += NT * U) {
        uint32_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = j0 + u * NT < n ? coherent_load(&row[j0 + u * NT]) : 0xFFFFFFFFu;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = j0 + u * NT;  // ascending j within the lane, so the first minimum is kept
            if (j < n && v[u] < best) {
                best = v[u];
                bi = j;
            }
        }
    }
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
        const uint32_t ov = __shfl_xor(best, m, kWave);
        const int oi = __shfl_xor(bi, m, kWave);
        if (ov < best || (ov == best && oi < bi)) {
            best = ov;
            bi = oi;
        }
    }
    const int lane = tid % kWave, wave = tid / kWave;
    if (lane == 0) {
        s_val[wave] = best;
        s_idx[wave] = bi;
    }
    __syncthreads();
    if (tid == 0) {
        for (int w = 1; w < NT / kWave; ++w)
            if (s_val[w] < best || (s_val[w] == best && s_idx[w] < bi)) {
                best = s_val[w];
                bi = s_idx[w];
            }
    }
    return bi;
}

}  // namespace ig
