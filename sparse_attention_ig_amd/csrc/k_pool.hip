// KV pool kernels (InfiniGen, arXiv 2406.19707, paper-graph-ui summary,
// section 3.4: "KV Cache Pool Management Under Memory Pressure" for the access
// counters and the victim, "Decoding Stage" step 5 for fetching the selected
// rows, "Prefill Stage" step 3 and "Partial Key Cache Updates During Decoding"
// for building and extending the partial key cache).
//
// Counters: one uint32 per pool slot and sequence.  k_touch runs one
// workgroup per sequence: it adds 1 per (head, selected slot) with integer
// atomics, so the result does not depend on the order of the additions; the
// atomics' return values tell whether any slot reached cmax (with counters
// below cmax on entry only a selected slot can), in which case the whole pool
// of that sequence is clamped and halved; the victim is the lowest index among
// the minima.  Keeping the whole sequence in one workgroup means the call
// needs no zeroed state and no second launch.
//
// Gather: 16-byte copies of whole rows; the source may be pinned host memory
// mapped into the device address space, in which case the reads travel over
// the host link (zero-copy) and the writes land in HBM.
#include <algorithm>

#include "ig_device.h"
#include "ig_internal.h"
#include "ig_pool_dev.h"

namespace ig {

constexpr int kTouchThreads = 1024;
constexpr int kTouchMaxHeads = 1024;
constexpr int kGatherThreads = 256;

// One workgroup per sequence: every (head, selected slot) of that sequence adds
// 1 with an integer atomic; an increment that returns cmax - 1 or more means
// the slot saturated (counters are below cmax on entry), in which case the
// whole pool of the sequence is clamped to cmax and halved.  Then the victim.
__global__ __launch_bounds__(kTouchThreads) void k_touch(uint32_t* __restrict__ C, const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ count, int H, int n, int n_cap,
                                                        int max_out, uint32_t cmax, int32_t* __restrict__ victim) {
    __shared__ int s_cnt[kTouchMaxHeads];
    __shared__ uint32_t s_val[kTouchThreads / kWave];
    __shared__ int s_idx[kTouchThreads / kWave];
    const int b = blockIdx.x, tid = threadIdx.x;
    uint32_t* row = C + static_cast<size_t>(b) * n_cap;
    for (int h = tid; h < H; h += kTouchThreads) s_cnt[h] = min(max(count[b * H + h], 0), max_out);
    __syncthreads();

    int sat = 0;
    const int total = H * max_out;
    constexpr int U = 8;  // index loads, then atomics, 8 per lane at a time, each batch issued together
    for (int e0 = tid; e0 < total; e0 += kTouchThreads * U) {
        int jj[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = e0 + u * kTouchThreads;
            const int h = e / max_out, i = e - h * max_out;
            jj[u] = (e < total && i < s_cnt[h]) ? idx[(static_cast<size_t>(b) * H + h) * max_out + i] : -1;
        }
        uint32_t old[U];
#pragma unroll
        for (int u = 0; u < U; ++u) old[u] = (jj[u] >= 0 && jj[u] < n) ? atomicAdd(&row[jj[u]], 1u) : 0u;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (jj[u] >= 0 && jj[u] < n && old[u] + 1u >= cmax) sat = 1;
    }
    sat = __syncthreads_or(sat);
    const int v = pool_finish<kTouchThreads>(row, n, cmax, sat != 0, victim != nullptr, s_val, s_idx);
    if (victim && tid == 0) victim[b] = v;
}

// Large selections: the increments spread over (b, h, chunk) workgroups; a slot that saturates sets
// its sequence's flag (zeroed first); a per-sequence finish halves if flagged and picks the victim.
__global__ __launch_bounds__(256) void k_touch_inc(uint32_t* __restrict__ C, const int32_t* __restrict__ idx,
                                                  const int32_t* __restrict__ count, int H, int n, int n_cap,
                                                  int max_out, uint32_t cmax, uint32_t* __restrict__ flags) {
    const int bh = blockIdx.y, b = bh / H;
    const int c = min(count[bh], max_out);
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < c) {
        const int j = idx[static_cast<size_t>(bh) * max_out + i];
        if (j >= 0 && j < n) {
            const uint32_t old = atomicAdd(&C[static_cast<size_t>(b) * n_cap + j], 1u);
            if (old + 1u >= cmax) flags[b] = 1u;
        }
    }
}

// Per-sequence finish: halve if flagged, pick the victim; the flag is returned to zero.
__global__ __launch_bounds__(kTouchThreads) void k_touch_finish(uint32_t* __restrict__ C, int n, int n_cap,
                                                               uint32_t cmax, uint32_t* __restrict__ flags,
                                                               int32_t* __restrict__ victim) {
    __shared__ uint32_t s_val[kTouchThreads / kWave];
    __shared__ int s_idx[kTouchThreads / kWave];
    const int b = blockIdx.x;
    const bool halve = flags[b] != 0u;
    const int v = pool_finish<kTouchThreads>(C + static_cast<size_t>(b) * n_cap, n, cmax, halve, victim != nullptr,
                                              s_val, s_idx);
    __syncthreads();  // every thread has read the flag
    if (threadIdx.x == 0) {
        if (victim) victim[b] = v;
        flags[b] = 0u;
    }
}

// Counters from the heads' selection bitmaps [B*H][ceil(n / 32)]: a workgroup owns 256 consecutive slots
// of sequence b (8 bitmap words per head).  It stages those words of every head in LDS (coalesced loads),
// then the thread of slot j adds the number of heads whose bit j is set to its counter (each slot has one
// owner: no atomics; the counters are read and written coalesced); a workgroup that saturated a slot
// flags its sequence for the finish.
constexpr int kBitsHeadsMax = 128;
__global__ __launch_bounds__(256) void k_touch_bits(uint32_t* __restrict__ C, const uint32_t* __restrict__ bits,
                                                   int H, int n, int n_cap, uint32_t cmax,
                                                   uint32_t* __restrict__ flags) {
    __shared__ uint32_t s_w[kBitsHeadsMax * 8];
    const int b = blockIdx.y, tid = threadIdx.x;
    const int nw = (n + 31) / 32;
    const int w0 = blockIdx.x * 8;
    for (int e = tid; e < H * 8; e += 256) {
        const int h = e / 8, w = w0 + e % 8;
        s_w[e] = w < nw ? bits[(static_cast<size_t>(b) * H + h) * nw + w] : 0u;
    }
    __syncthreads();
    const int j = blockIdx.x * 256 + tid;
    int sat = 0;
    if (j < n) {
        uint32_t inc = 0;
        const uint32_t* col = s_w + tid / 32;
        for (int h = 0; h < H; ++h) inc += (col[h * 8] >> (tid & 31)) & 1u;
        if (inc) {
            uint32_t* c = C + static_cast<size_t>(b) * n_cap + j;
            const uint32_t v = *c + inc;
            *c = v;
            sat = v >= cmax ? 1 : 0;
        }
    }
    if (__syncthreads_or(sat) && tid == 0) atomicOr(&flags[b], 1u);
}

int launch_touch_bits(uint32_t* counters, const uint32_t* bits, int B, int H, int n, int n_cap, uint32_t cmax,
                      uint32_t* flags, int32_t* victim, hipStream_t s) {
    hipLaunchKernelGGL(k_touch_bits, dim3((n + 255) / 256, B), dim3(256), 0, s, counters, bits, H, n, n_cap, cmax,
                       flags);
    const int e = static_cast<int>(hipGetLastError());
    if (e) return e;
    hipLaunchKernelGGL(k_touch_finish, dim3(B), dim3(kTouchThreads), 0, s, counters, n, n_cap, cmax, flags, victim);
    return static_cast<int>(hipGetLastError());
}

size_t touch_ws_bytes(int B) { return ((static_cast<size_t>(B) * sizeof(uint32_t) + 255) / 256) * 256; }

bool touch_single_kernel(int H, int max_out) { return static_cast<int64_t>(H) * max_out <= 32768; }

int launch_touch(uint32_t* counters, const int32_t* idx, const int32_t* count, int B, int H, int n, int n_cap,
                 int max_out, uint32_t cmax, int32_t* victim, void* ws, hipStream_t s) {
    if (touch_single_kernel(H, max_out)) {
        hipLaunchKernelGGL(k_touch, dim3(B), dim3(kTouchThreads), 0, s, counters, idx, count, H, n, n_cap, max_out,
                           cmax, victim);
        return static_cast<int>(hipGetLastError());
    }
    uint32_t* flags = static_cast<uint32_t*>(ws);
    int e = launch_zero(flags, static_cast<size_t>(B) * sizeof(uint32_t), s);
    if (e) return e;
    hipLaunchKernelGGL(k_touch_inc, dim3((max_out + 255) / 256, B * H), dim3(256), 0, s, counters, idx, count, H, n,
                       n_cap, max_out, cmax, flags);
    e = static_cast<int>(hipGetLastError());
    if (e) return e;
    hipLaunchKernelGGL(k_touch_finish, dim3(B), dim3(kTouchThreads), 0, s, counters, n, n_cap, cmax, flags, victim);
    return static_cast<int>(hipGetLastError());
}

// rows of RB bytes (RB % 16 == 0), LPR = RB / 16 lanes per row.  The work is cut into units of
// kGatherRows rows of one (b, h); the workgroups walk the units (workgroup w takes units w, w + gridDim.x,
// ..).  A gather from host memory runs at most kGatherHostWgs workgroups: the host link needs only enough
// reads in flight to cover its latency, and the rest of the GPU stays free for kernels on other streams
// (a flood of slow host reads holds them back); a gather from device memory runs one workgroup per unit.
// Every lane issues the loads of all its rows of a unit before any store.
constexpr int kGatherRows = 64;
constexpr int kGatherHostWgs = 128;

// Whether p points to host memory (pinned, mapped into the device's address space); pointers the runtime
// does not know count as host memory.
bool host_resident(const void* p) {
    hipPointerAttribute_t a{};
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError();  // (not a launch error)
        return true;
    }
    return a.type != hipMemoryTypeDevice;
}
__global__ __launch_bounds__(kGatherThreads) void k_gather(const char* __restrict__ K, const char* __restrict__ V,
                                                          const int32_t* __restrict__ idx,
                                                          const int32_t* __restrict__ count, int row_bytes,
                                                          int n_cap, int max_out, int chunks, int64_t units,
                                                          char* __restrict__ Kc, char* __restrict__ Vc) {
    constexpr int U = kGatherRows / (kGatherThreads / 16);  // rows per lane and unit at the widest row
    const int lpr = row_bytes / 16;
    const int rows_per_step = kGatherThreads / lpr;
    const int li = threadIdx.x % lpr, ri = threadIdx.x / lpr;
    if (ri >= rows_per_step) return;
    for (int64_t u0 = blockIdx.x; u0 < units; u0 += gridDim.x) {
        const int64_t bh = u0 / chunks;
        const int chunk = static_cast<int>(u0 - bh * chunks);
        const int c = min(count[bh], max_out);
        const int i0 = chunk * kGatherRows;
        const int i1 = min(c, i0 + kGatherRows);
        const size_t src_head = static_cast<size_t>(bh) * n_cap * row_bytes;
        const size_t dst_head = static_cast<size_t>(bh) * max_out * row_bytes;
        for (int ib = i0 + ri; ib < i1; ib += rows_per_step * U) {
            int j[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = ib + u * rows_per_step;
                j[u] = i < i1 ? min(max(idx[static_cast<size_t>(bh) * max_out + i], 0), n_cap - 1) : -1;
            }
            uint4 kv[U], vv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (j[u] >= 0) {
                    const size_t so = src_head + static_cast<size_t>(j[u]) * row_bytes + li * 16;
                    kv[u] = load_raw16(K + so);
                    vv[u] = load_raw16(V + so);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (j[u] >= 0) {
                    const size_t dof = dst_head + static_cast<size_t>(ib + u * rows_per_step) * row_bytes + li * 16;
                    store_raw16(Kc + dof, kv[u]);
                    store_raw16(Vc + dof, vv[u]);
                }
            }
        }
    }
}

int launch_gather(const void* K, const void* V, const int32_t* idx, const int32_t* count, int B, int H, int d,
                  int n_cap, int max_out, int dtype, void* Kc, void* Vc, hipStream_t s) {
    const int row_bytes = d * (dtype == IG_BF16 ? 2 : 4);
    const int chunks = (max_out + kGatherRows - 1) / kGatherRows;
    const int64_t units = static_cast<int64_t>(chunks) * B * H;
    const int grid = static_cast<int>(std::min<int64_t>(units, host_resident(K) ? kGatherHostWgs : (1 << 30)));
    hipLaunchKernelGGL(k_gather, dim3(grid), dim3(kGatherThreads), 0, s, static_cast<const char*>(K),
                       static_cast<const char*>(V), idx, count, row_bytes, n_cap, max_out, chunks, units,
                       static_cast<char*>(Kc), static_cast<char*>(Vc));
    return static_cast<int>(hipGetLastError());
}

template <typename T>
__global__ __launch_bounds__(256) void k_build_partial(const T* __restrict__ K, const int32_t* __restrict__ chan,
                                                      T* __restrict__ Kp, int H, int d, int r, int n_cap, int row0,
                                                      int row1) {
    const int bh = blockIdx.y, h = bh % H;
    const int64_t e0 = static_cast<int64_t>(blockIdx.x) * 256 * 4;
    const int64_t total = static_cast<int64_t>(row1 - row0) * r;
    for (int u = 0; u < 4; ++u) {
        const int64_t e = e0 + u * 256 + threadIdx.x;
        if (e >= total) return;
        const int j = row0 + static_cast<int>(e / r), c = static_cast<int>(e % r);
        const int ch = min(max(chan[h * r + c], 0), d - 1);
        Kp[(static_cast<size_t>(bh) * n_cap + j) * r + c] = K[(static_cast<size_t>(bh) * n_cap + j) * d + ch];
    }
}

int launch_build_partial(const void* K, const int32_t* chan, void* Kp, int B, int H, int d, int r, int n_cap,
                         int row0, int row1, int dtype, hipStream_t s) {
    const int64_t total = static_cast<int64_t>(row1 - row0) * r;
    const dim3 grid(static_cast<unsigned>((total + 1023) / 1024), B * H);
    if (dtype == IG_BF16)
        hipLaunchKernelGGL((k_build_partial<uint16_t>), grid, dim3(256), 0, s, static_cast<const uint16_t*>(K), chan,
                           static_cast<uint16_t*>(Kp), H, d, r, n_cap, row0, row1);
    else
        hipLaunchKernelGGL((k_build_partial<float>), grid, dim3(256), 0, s, static_cast<const float*>(K), chan,
                           static_cast<float*>(Kp), H, d, r, n_cap, row0, row1);
    return static_cast<int>(hipGetLastError());
}

template <typename T>
__global__ __launch_bounds__(256) void k_append(T* __restrict__ K, T* __restrict__ V, T* __restrict__ Kp,
                                               uint32_t* __restrict__ C, const int32_t* __restrict__ chan,
                                               const T* __restrict__ k_new, const T* __restrict__ v_new,
                                               const int32_t* __restrict__ victim, int H, int d, int r, int n_cap,
                                               int n, int32_t* __restrict__ slot_out) {
    const int bh = blockIdx.x, b = bh / H, h = bh - b * H;
    int slot = n < n_cap ? n : victim[b];
    slot = min(max(slot, 0), n_cap - 1);
    const size_t row = (static_cast<size_t>(bh) * n_cap + slot);
    for (int t = threadIdx.x; K && t < d; t += 256) {  // (no full rows: a quantised pool takes them)
        K[row * d + t] = k_new[static_cast<size_t>(bh) * d + t];
        V[row * d + t] = v_new[static_cast<size_t>(bh) * d + t];
    }
    for (int c = threadIdx.x; c < r; c += 256)
        Kp[row * r + c] = k_new[static_cast<size_t>(bh) * d + min(max(chan[h * r + c], 0), d - 1)];
    if (h == 0 && threadIdx.x == 0) {
        if (C) C[static_cast<size_t>(b) * n_cap + slot] = 0u;
        if (slot_out) slot_out[b] = slot;
    }
}

int launch_append(void* K, void* V, void* Kp, uint32_t* counters, const int32_t* chan, const void* k_new,
                  const void* v_new, const int32_t* victim, int B, int H, int d, int r, int n_cap, int n, int dtype,
                  int32_t* slot_out, hipStream_t s) {
    if (dtype == IG_BF16)
        hipLaunchKernelGGL((k_append<uint16_t>), dim3(B * H), dim3(256), 0, s, static_cast<uint16_t*>(K),
                           static_cast<uint16_t*>(V), static_cast<uint16_t*>(Kp), counters, chan,
                           static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), victim, H, d, r,
                           n_cap, n, slot_out);
    else
        hipLaunchKernelGGL((k_append<float>), dim3(B * H), dim3(256), 0, s, static_cast<float*>(K),
                           static_cast<float*>(V), static_cast<float*>(Kp), counters, chan,
                           static_cast<const float*>(k_new), static_cast<const float*>(v_new), victim, H, d, r, n_cap,
                           n, slot_out);
    return static_cast<int>(hipGetLastError());
}

}  // namespace ig
