// topk.hip -- exact top-k selection of float logits on gfx950.
//
// For each row the candidates are the entries before n_valid whose value is
// neither NaN nor -inf; the k largest are kept, equal values going to the
// lower index, and their indices are written in ascending order, padded
// with -1 (the index top-k of "perf(kernel): keep 16-byte kv loads in dsv4
// sparse attention and unroll gated pool", Kernel time).
//
// Values become order-preserving 32-bit keys (0 = not a candidate).  One
// workgroup selects the top-k of one segment with a 4-pass, 8-bit radix
// select over keys held in registers (LDS histograms, one wave scanning the
// 256 bins), then takes the keys above the threshold plus the first
// threshold-equal keys in index order (block prefix sums keep index order,
// which is also the tie-break).  Pass 1 cuts each row into 4096-entry
// segments and writes each segment's survivors (key, index) to a slot of k
// entries; later passes merge groups of slots the same way until one slot is
// left, which writes the final index list.  The top-k of a union is always
// inside the union of the parts' top-k under the same total order, so every
// pass is exact.
#include "common.hpp"
#include "internal.hpp"

namespace sap {
namespace {

constexpr int kThreads = 256;
constexpr int kRowSeg = 4096;            // pass-1 segment (16 per thread)
constexpr int kMergeSeg = 16384;         // later passes (64 per thread)

__device__ __forceinline__ uint32_t order_key(float v)
{
    const uint32_t u = __float_as_uint(v);
    if (v != v || u == 0xFF800000u) return 0u;          // NaN, -inf: not candidates
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // >= 0x00800000 otherwise
}

struct PassParams {
    int B, k;
    // pass 1 input: a row of floats
    const float *x;
    int64_t x_sb;
    const int32_t *n_valid;
    int N;
    // later-pass input: slots of k (key, index) pairs with counts
    const uint32_t *in_key;
    const int32_t *in_idx;
    const int32_t *in_cnt;
    int in_slots, slots_per_wg;
    // output: either slots or the final list
    uint32_t *out_key;
    int32_t *out_idx;
    int32_t *out_cnt;
    int out_slots;
    int32_t *final_out;
    int64_t final_sb;
};

__device__ __forceinline__ int wave_incl_scan(int x, int lane)
{
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(x, off, kWave);
        if (lane >= off) x += y;
    }
    return x;
}

// exclusive prefix over the block in thread order; `total` gets the sum
__device__ __forceinline__ int block_excl_scan(int v, int *sh, int &total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int inc = wave_incl_scan(v, lane);
    if (lane == 63) sh[wave] = inc;
    __syncthreads();
    int base = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) {
        const int s = sh[w];
        if (w < wave) base += s;
        total += s;
    }
    __syncthreads();
    return base + inc - v;
}

template <int PER, bool FROM_ROW>
__global__ __launch_bounds__(kThreads) void topk_pass_kernel(PassParams p)
{
    __shared__ uint32_t hist[256];
    __shared__ int sh[8];
    const int b = blockIdx.y, seg = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;

    // this thread's contiguous run of segment positions [tid*PER, tid*PER+PER)
    uint32_t key[PER];
    int32_t ind[PER];
    if constexpr (FROM_ROW) {
        int nv = p.n_valid ? p.n_valid[b] : p.N;
        nv = min(max(nv, 0), p.N);
        const int64_t base = (int64_t)seg * (kThreads * PER);
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int64_t i = base + (int64_t)tid * PER + j;
            ind[j] = (int32_t)i;
            key[j] = i < nv ? order_key(p.x[(int64_t)b * p.x_sb + i]) : 0u;
        }
    } else {
        const int s0 = seg * p.slots_per_wg;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int pos = tid * PER + j;
            const int s = s0 + pos / p.k;
            const int e = pos - (pos / p.k) * p.k;
            key[j] = 0u;
            ind[j] = -1;
            if (s < p.in_slots && s < s0 + p.slots_per_wg) {
                const int64_t slot = (int64_t)b * p.in_slots + s;
                if (e < p.in_cnt[slot]) {
                    key[j] = p.in_key[slot * p.k + e];
                    ind[j] = p.in_idx[slot * p.k + e];
                }
            }
        }
    }

    int cnt = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) cnt += key[j] != 0u;
    int n_cand;
    (void)block_excl_scan(cnt, sh, n_cand);
    const int kk = min(p.k, n_cand);

    uint32_t T = 0xFFFFFFFFu;
    int need_eq = 0;
    if (kk > 0) {
        uint32_t prefix = 0u, mask = 0u;
        int rem = kk;
        for (int shift = 24; shift >= 0; shift -= 8) {
            hist[tid] = 0u;
            __syncthreads();
#pragma unroll
            for (int j = 0; j < PER; ++j)
                if (key[j] != 0u && (key[j] & mask) == prefix) atomicAdd(&hist[(key[j] >> shift) & 255u], 1u);
            __syncthreads();
            if (wave == 0) {
                const int c = (int)(hist[4 * lane] + hist[4 * lane + 1] + hist[4 * lane + 2] + hist[4 * lane + 3]);
                // suffix sum over lanes: entries in bins >= 4*lane
                int x = c;
#pragma unroll
                for (int off = 1; off < kWave; off <<= 1) {
                    const int y = __shfl_down(x, off, kWave);
                    if (lane + off < kWave) x += y;
                }
                if (x >= rem && x - c < rem) {
                    int above = x - c;
                    int bin = 4 * lane;
                    for (int bb = 4 * lane + 3; bb >= 4 * lane; --bb) {
                        if (above + (int)hist[bb] >= rem) { bin = bb; break; }
                        above += (int)hist[bb];
                    }
                    sh[4] = bin;
                    sh[5] = above;
                }
            }
            __syncthreads();
            const int bin = sh[4];
            rem -= sh[5];
            prefix |= (uint32_t)bin << shift;
            mask |= 255u << shift;
            __syncthreads();
        }
        T = prefix;
        need_eq = rem;
    }

    int gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        gt += (kk > 0 && key[j] > T);
        eq += (kk > 0 && key[j] == T);
    }
    int tot;
    const int eq_before = block_excl_scan(eq, sh, tot);
    const int take_eq = max(0, min(eq, need_eq - eq_before));
    int n_out;
    int pos = block_excl_scan(gt + take_eq, sh, n_out);

    if (p.final_out) {
        int32_t *o = p.final_out + (int64_t)b * p.final_sb;
        int seen = 0;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const bool sel = kk > 0 && (key[j] > T || (key[j] == T && seen++ < take_eq));
            if (sel) o[pos++] = ind[j];
        }
        for (int i = n_out + tid; i < p.k; i += kThreads) o[i] = -1;
    } else {
        const int64_t slot = (int64_t)b * p.out_slots + seg;
        uint32_t *ok = p.out_key + slot * p.k;
        int32_t *oi = p.out_idx + slot * p.k;
        int seen = 0;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const bool sel = kk > 0 && (key[j] > T || (key[j] == T && seen++ < take_eq));
            if (sel) {
                ok[pos] = key[j];
                oi[pos] = ind[j];
                ++pos;
            }
        }
        if (tid == 0) p.out_cnt[slot] = n_out;
    }
}

}  // namespace

// Workspace: two slot buffers sized for pass 1 (ceil(N/4096) slots per row).
size_t topk_slot_bytes(int B, int N, int k)
{
    const int64_t slots = N > kRowSeg ? (N + kRowSeg - 1) / kRowSeg : 0;
    const int64_t per = (int64_t)B * slots * ((int64_t)k * 8 + 4);
    return (size_t)((per + 255) / 256 * 256);
}

hipError_t launch_topk(const TopkParams &tp, hipStream_t s)
{
    if (tp.B == 0) return hipSuccess;
    PassParams p{};
    p.B = tp.B;
    p.k = tp.k;
    p.x = tp.x;
    p.x_sb = tp.x_sb;
    p.n_valid = tp.n_valid;
    p.N = tp.N;
    const int slots1 = tp.N > kRowSeg ? (tp.N + kRowSeg - 1) / kRowSeg : 1;
    if (slots1 == 1) {
        p.final_out = tp.out;
        p.final_sb = tp.out_sb;
        hipLaunchKernelGGL((topk_pass_kernel<kRowSeg / kThreads, true>), dim3(1, tp.B), dim3(kThreads), 0, s, p);
        return hipGetLastError();
    }
    // ping-pong slot buffers inside the workspace
    const size_t half = topk_slot_bytes(tp.B, tp.N, tp.k);
    uint8_t *buf[2] = {(uint8_t *)tp.workspace, (uint8_t *)tp.workspace + half};
    struct Slots { uint32_t *key; int32_t *idx; int32_t *cnt; };
    auto carve = [&](uint8_t *base, int slots) {
        Slots r;
        r.key = (uint32_t *)base;
        r.idx = (int32_t *)(base + (size_t)tp.B * slots * tp.k * 4);
        r.cnt = (int32_t *)(base + (size_t)tp.B * slots * tp.k * 8);
        return r;
    };
    {
        const Slots o = carve(buf[0], slots1);
        p.out_key = o.key;
        p.out_idx = o.idx;
        p.out_cnt = o.cnt;
    }
    p.out_slots = slots1;
    hipLaunchKernelGGL((topk_pass_kernel<kRowSeg / kThreads, true>), dim3(slots1, tp.B), dim3(kThreads), 0, s, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;

    int in_slots = slots1, cur = 0;
    const int spw = kMergeSeg / tp.k;                 // slots merged per workgroup (>= 4)
    while (true) {
        PassParams q{};
        q.B = tp.B;
        q.k = tp.k;
        const Slots in = carve(buf[cur], in_slots);
        q.in_key = in.key;
        q.in_idx = in.idx;
        q.in_cnt = in.cnt;
        q.in_slots = in_slots;
        q.slots_per_wg = spw;
        const int out_slots = (in_slots + spw - 1) / spw;
        if (out_slots == 1) {
            q.final_out = tp.out;
            q.final_sb = tp.out_sb;
        } else {
            const Slots o = carve(buf[cur ^ 1], out_slots);
            q.out_key = o.key;
            q.out_idx = o.idx;
            q.out_cnt = o.cnt;
            q.out_slots = out_slots;
        }
        hipLaunchKernelGGL((topk_pass_kernel<kMergeSeg / kThreads, false>), dim3(out_slots, tp.B), dim3(kThreads), 0,
                           s, q);
        err = hipGetLastError();
        if (err != hipSuccess || out_slots == 1) return err;
        in_slots = out_slots;
        cur ^= 1;
    }
}

}  // namespace sap
