// index_build.hip -- logical window positions and compressed entries to
// physical pool rows through page tables (the column set of "perf(kernel):
// keep 16-byte kv loads in dsv4 sparse attention and unroll gated pool":
// a causal sliding window plus the selected compressed entries).
#include "internal.hpp"

namespace sap {
namespace {

__global__ __launch_bounds__(256) void build_idx_kernel(IdxBuildParams p)
{
    const int t = blockIdx.x;
    const int C = p.n_win + p.n_cmp;
    const int s = p.seq[t];
    const int pos = p.pos[t];
    for (int c = blockIdx.y * blockDim.x + threadIdx.x; c < C; c += gridDim.y * blockDim.x) {
        int32_t r = -1;
        if (c < p.n_win) {
            const int64_t q = (int64_t)pos - (p.n_win - 1) + c;
            if (q >= 0) r = p.win_pt[(int64_t)s * p.win_pt_sb + q / p.page] * p.page + (int32_t)(q % p.page);
        } else {
            const int32_t L = p.cmp_logical[(int64_t)t * p.cmp_logical_st + (c - p.n_win)];
            if (L >= 0) r = p.cmp_pt[(int64_t)s * p.cmp_pt_sb + L / p.page] * p.page + L % p.page;
        }
        p.idx[(int64_t)t * p.idx_st + c] = r;
    }
}

}  // namespace

hipError_t launch_build_idx(const IdxBuildParams &p, hipStream_t s)
{
    const int C = p.n_win + p.n_cmp;
    const unsigned gy = (unsigned)((C + 255) / 256);
    hipLaunchKernelGGL(build_idx_kernel, dim3((unsigned)p.T, gy), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace sap
