// Standalone sparse decode attention (InfiniGen, arXiv 2406.19707,
// paper-graph-ui summary, section 3.2 Inference Controller; section 2,
// softmax(QK^T)V over the cached rows): one 256-thread workgroup per (split,
// b, h) running attn_item, then the split combine when a (b, h) is split.
// Split-K: when there are too few (b, h) units to fill the chip, the selected
// rows of one (b, h) are cut into splits of at least 128 rows.
#include "ig_attn_dev.h"
#include "ig_internal.h"

namespace ig {

constexpr int kAttnThreads = 256;

template <typename T, int LPR>
__global__ __launch_bounds__(kAttnThreads) void k_attn_split(AttnArgs a) {
    __shared__ AttnShared<kAttnThreads, LPR, Vec<T>::N> sm;
    attn_item<T, LPR, kAttnThreads>(a, blockIdx.y, blockIdx.x, sm);
}

__global__ __launch_bounds__(256) void k_attn_combine(const float* __restrict__ part, int nsplit, int d,
                                                      float* __restrict__ out, float* __restrict__ lse) {
    combine_item(CombineArgs{part, nsplit, d, out, lse}, blockIdx.x);
}

AttnPlan plan_attn(int B, int H, int d, int max_out) {
    AttnPlan p{};
    const int64_t bh = static_cast<int64_t>(B) * H;
    // one workgroup per (b, h) when there are enough of them to fill the chip; otherwise split the
    // selected rows so that about 768 workgroups run (three per CU: the last ones to start are short
    // enough not to trail the rest; measured against 512 and 1024), each with at least 128 rows
    int64_t nsplit = 1;
    if (bh < 256) {
        nsplit = (768 + bh - 1) / bh;
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
    const AttnArgs a{q, K, V, ld_rows, idx, count, d, max_out, p.rows_per_split, p.nsplit, scale, out, lse, part};
#define IG_ATTN_CASE(L)                                                                     \
    case L:                                                                                 \
        hipLaunchKernelGGL((k_attn_split<T, L>), grid, dim3(kAttnThreads), 0, s, a);       \
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
    return launch_attn_combine(part, p.nsplit, d, B * H, out, lse, s);
}

int launch_attn_combine(const float* part, int nsplit, int d, int BH, float* out, float* lse, hipStream_t s) {
    hipLaunchKernelGGL(k_attn_combine, dim3(BH), dim3(std::min(256, d)), 0, s, part, nsplit, d, out, lse);
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
