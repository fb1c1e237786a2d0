// Device-side partial weight index generation (InfiniGen, arXiv 2406.19707,
// paper-graph-ui summary, section 3.4 "Prefill Stage: Partial Weight Index
// Generation", steps 2-3): per head, the r channels with the largest
// column sums of |W~_Q| plus |K~| over the prefilled rows, and the partial
// query weight packed one row per chosen channel.  Same result as the host
// routine (float64 sums, ties to the lower channel, channels ascending); the
// sums are taken in a fixed order, so the result is deterministic.
//
//   k_colsum_w   |W~_Q| column sums over D-row slices -> partials [slices][H*d]
//   k_colsum_k   |K~| column sums over (b, h, row chunk) -> partials [B*chunks][H][d]
//   k_pick       per head: add the partials in order, rank the channels, write chan
//   k_pack_wq    Wq_part[h*r + k][i] = Wq_s[i][h*d + chan[h][k]] through an LDS tile
#include <cmath>

#include "ig_device.h"
#include "ig_internal.h"

namespace ig {

constexpr int kSetupThreads = 256;
constexpr int kColRows = 64;      // W rows per slice of k_colsum_w
constexpr int kKRows = 256;       // cache rows per chunk of k_colsum_k

__device__ __forceinline__ double abs_elem(const float* p, size_t i) { return fabs(static_cast<double>(p[i])); }
__device__ __forceinline__ double abs_elem(const uint16_t* p, size_t i) {
    return fabs(static_cast<double>(bf16_to_f32(p[i])));
}

// one column per thread, kColRows rows per workgroup (loads of a row are coalesced across threads)
template <typename T>
__global__ __launch_bounds__(kSetupThreads) void k_colsum_w(const T* __restrict__ W, int D, int ncol,
                                                            double* __restrict__ part) {
    const int c = blockIdx.x * kSetupThreads + threadIdx.x;
    const int i0 = blockIdx.y * kColRows;
    if (c >= ncol) return;
    double s = 0.0;
    constexpr int U = 8;
    for (int i = i0; i < min(D, i0 + kColRows); i += U) {
        double v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = i + u < D && i + u < i0 + kColRows ? abs_elem(W, static_cast<size_t>(i + u) * ncol + c) : 0.0;
#pragma unroll
        for (int u = 0; u < U; ++u) s += v[u];
    }
    part[static_cast<size_t>(blockIdx.y) * ncol + c] = s;
}

// workgroup (row chunk, b*H + h): thread t sums channel t % d over rows j = t / d, t / d + 256 / d, ...
template <typename T>
__global__ __launch_bounds__(kSetupThreads) void k_colsum_k(const T* __restrict__ K, int H, int d, int n_cap, int n,
                                                            int chunks, double* __restrict__ part) {
    __shared__ double red[kSetupThreads];
    const int bh = blockIdx.y, b = bh / H, h = bh - b * H;
    const int tid = threadIdx.x;
    const int c = tid % d, g = tid / d, G = kSetupThreads / d;  // d divides 256 (d a power of two <= 256)
    const int j0 = blockIdx.x * kKRows, j1 = min(n, j0 + kKRows);
    const T* row = K + static_cast<size_t>(bh) * n_cap * d;
    double s = 0.0;
    for (int j = j0 + g; j < j1; j += G) s += abs_elem(row, static_cast<size_t>(j) * d + c);
    red[tid] = s;
    __syncthreads();
    if (tid < d) {
        double t = 0.0;
        for (int k = 0; k < G; ++k) t += red[k * d + tid];
        part[((static_cast<size_t>(b) * chunks + blockIdx.x) * H + h) * d + tid] = t;
    }
}

// one workgroup per head: score[c] = sum of the W partials + sum of the K partials (fixed order);
// channel c is chosen if fewer than r channels rank above it (larger score, or equal and lower index)
__global__ __launch_bounds__(kSetupThreads) void k_pick(const double* __restrict__ wpart, int wslices,
                                                       const double* __restrict__ kpart, int kparts, int H, int d,
                                                       int r, int32_t* __restrict__ chan) {
    __shared__ double sc[kSetupThreads];
    __shared__ int chosen[kSetupThreads];
    const int h = blockIdx.x, c = threadIdx.x;
    const int ncol = H * d;
    if (c < d) {
        double s = 0.0;
        for (int k = 0; k < wslices; ++k) s += wpart[static_cast<size_t>(k) * ncol + h * d + c];
        double t = 0.0;
        for (int k = 0; k < kparts; ++k) t += kpart[(static_cast<size_t>(k) * H + h) * d + c];
        sc[c] = s + t;
    }
    __syncthreads();
    int rank = 0;
    if (c < d) {
        const double v = sc[c];
        for (int o = 0; o < d; ++o) rank += (sc[o] > v || (sc[o] == v && o < c)) ? 1 : 0;
        chosen[c] = rank < r ? 1 : 0;
    }
    __syncthreads();
    if (c < d && chosen[c]) {
        int pos = 0;  // ascending channel order
        for (int o = 0; o < c; ++o) pos += chosen[o];
        chan[h * r + pos] = c;
    }
}

// workgroup (64-row tile of D, head h): the head's d columns of 64 rows go to LDS, then each chosen
// channel's 64 values are written as one contiguous piece of its Wq_part row
template <typename T>
__global__ __launch_bounds__(kSetupThreads) void k_pack_wq(const T* __restrict__ W, int D, int H, int d, int r,
                                                          const int32_t* __restrict__ chan, T* __restrict__ Wp) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    T* tile = reinterpret_cast<T*>(smem_raw);  // [64][d]
    const int i0 = blockIdx.x * 64, h = blockIdx.y, tid = threadIdx.x;
    const int rows = min(64, D - i0);
    const size_t ncol = static_cast<size_t>(H) * d;
    for (int e = tid; e < rows * d; e += kSetupThreads) {
        const int i = e / d, c = e - i * d;
        tile[e] = W[static_cast<size_t>(i0 + i) * ncol + static_cast<size_t>(h) * d + c];
    }
    __syncthreads();
    for (int e = tid; e < r * rows; e += kSetupThreads) {
        const int k = e / rows, i = e - k * rows;
        const int c = min(max(chan[h * r + k], 0), d - 1);
        Wp[(static_cast<size_t>(h) * r + k) * D + i0 + i] = tile[i * d + c];
    }
}

SetupPlan plan_setup(int B, int H, int d, int D, int n) {
    SetupPlan p{};
    p.wslices = (D + kColRows - 1) / kColRows;
    p.kchunks = (n + kKRows - 1) / kKRows;
    p.off_k = (static_cast<size_t>(p.wslices) * H * d * sizeof(double) + 255) / 256 * 256;
    p.ws_bytes = p.off_k + static_cast<size_t>(B) * p.kchunks * H * d * sizeof(double);
    return p;
}

template <typename T>
static int launch_setup_t(const T* Wq_s, int D, int H, int d, int r, const T* K_s, int B, int n_cap, int n,
                          int32_t* chan, T* Wq_part, void* ws, hipStream_t s) {
    const SetupPlan p = plan_setup(B, H, d, D, n);
    double* wpart = static_cast<double*>(ws);
    double* kpart = reinterpret_cast<double*>(static_cast<char*>(ws) + p.off_k);
    const int ncol = H * d;
    hipLaunchKernelGGL(k_colsum_w<T>, dim3((ncol + kSetupThreads - 1) / kSetupThreads, p.wslices), dim3(kSetupThreads),
                       0, s, Wq_s, D, ncol, wpart);
    int e = static_cast<int>(hipGetLastError());
    if (e) return e;
    hipLaunchKernelGGL(k_colsum_k<T>, dim3(p.kchunks, B * H), dim3(kSetupThreads), 0, s, K_s, H, d, n_cap, n,
                       p.kchunks, kpart);
    if ((e = static_cast<int>(hipGetLastError()))) return e;
    hipLaunchKernelGGL(k_pick, dim3(H), dim3(kSetupThreads), 0, s, wpart, p.wslices, kpart, B * p.kchunks, H, d, r,
                       chan);
    if ((e = static_cast<int>(hipGetLastError()))) return e;
    hipLaunchKernelGGL(k_pack_wq<T>, dim3((D + 63) / 64, H), dim3(kSetupThreads), 64 * d * sizeof(T), s, Wq_s, D, H,
                       d, r, chan, Wq_part);
    return static_cast<int>(hipGetLastError());
}

int launch_setup(const void* Wq_s, int D, int H, int d, int r, const void* K_s, int B, int n_cap, int n, int dtype,
                 int32_t* chan, void* Wq_part, void* ws, hipStream_t s) {
    if (dtype == IG_BF16)
        return launch_setup_t(static_cast<const uint16_t*>(Wq_s), D, H, d, r, static_cast<const uint16_t*>(K_s), B,
                              n_cap, n, chan, static_cast<uint16_t*>(Wq_part), ws, s);
    return launch_setup_t(static_cast<const float*>(Wq_s), D, H, d, r, static_cast<const float*>(K_s), B, n_cap, n,
                          chan, static_cast<float*>(Wq_part), ws, s);
}

}  // namespace ig
