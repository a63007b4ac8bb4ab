// topk.hip -- exact top-k selection of float logits on gfx950.
//
// For each row the candidates are the entries before n_valid whose value is
// neither NaN nor -inf; the k largest are kept, equal values going to the
// lower index, and their indices are written in ascending order, padded
// with -1 (the index top-k of "perf(kernel): keep 16-byte kv loads in dsv4
// sparse attention and unroll gated pool", Kernel time).
//
// Values become order-preserving 32-bit keys (0 = not a candidate).  The
// selection core runs in one 1024-thread workgroup (one CU) on keys held in
// registers.  One CU issues 64 lane-operations per cycle, so at 8192 keys
// every instruction per key costs 128 cycles: the core is built to spend few
// instructions per key, not to save barriers.
//  - radix select finds the prefix of the k-th largest key.  It starts below
//    the bits every candidate shares (found by AND/OR reductions, which also
//    tell whether any key is a non-candidate; if none is, the first pass
//    needs no prefix test), takes 11 bits per pass into one LDS histogram of
//    2048 bins, finds the bin holding the k-th key in one wave with two DPP
//    scans, and stops as soon as that bin is taken whole;
//  - keys sit in a strided layout (thread t holds entries j*1024 + t), so a
//    ballot over one key column lists 64 consecutive entries in order: a
//    selected key's output slot is the count of selected keys in earlier
//    (column, wave) pairs, from one exchange of per-pair ballot counts, plus
//    mbcnt of its ballot.  The output is in ascending index order -- no sort.
// Wave-level scans and reductions use DPP row shifts and broadcasts.
// Rows of up to 16384 entries are selected directly.  Longer rows take two
// launches: a filter launch where each workgroup derives the same threshold
// from a fixed strided sample of the row and compacts the keys of its 4096
// positions at or above it into its own slot, then a select launch that
// gathers the slots (in position order) and runs the core on them.  If the
// sample's threshold was too high (fewer than k keys at or above it) or a
// slot overflowed, the select launch falls back to radix select over the row
// streamed from memory -- slower, never wrong.
#include "common.hpp"
#include "internal.hpp"

#include <type_traits>

namespace sap {
namespace {

constexpr int kT = 1024;                 // threads per workgroup
constexpr int kW = kT / kWave;           // waves per workgroup
constexpr int kDirectMax = 16384;        // rows selected in one launch (16 keys per thread)
constexpr int kChunk = 4096;             // positions per filter workgroup (4 keys per thread)
constexpr int kSlotCap = 2048;           // candidates one filter workgroup may keep
constexpr int kMaxChunks = 4096;         // two-launch path: N <= kChunk * kMaxChunks
constexpr int kSample = 4096;            // strided sample that sets the filter threshold
constexpr int kMaxK = 4096;

__device__ __forceinline__ uint32_t order_key(float v)
{
    // v + 0 turns -0.0 into +0.0 (equal values share one key) and leaves every
    // other value as it is; negative values have all bits flipped, others only
    // the sign bit.  Keys of candidates are >= 0x00800000.
    const uint32_t u = __float_as_uint(v + 0.0f);
    const uint32_t key = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
    return __builtin_amdgcn_classf(v, 0x7) ? 0u : key;   // signaling or quiet NaN, -inf
}

// Radix select keeps one 2048-bin LDS histogram, counting the keys inside
// the current prefix.
constexpr int kBins = 2048;

constexpr int kMaxKPT = 16;   // keys per thread of the selection core

struct Shared {
    __attribute__((aligned(16))) uint32_t hist[kBins];
    int red[kW];
    uint32_t wand[kW], wor[kW], wzero[kW];
    __attribute__((aligned(16))) int misc[4];
    __attribute__((aligned(16))) int tab[kMaxKPT * kW];   // per (key column, wave) counts
};

// exclusive prefix sum over the workgroup in thread order; total to all
__device__ int block_excl_scan(int v, Shared &s, int &total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int x = wave_incl_sum(v);
    if (lane == 63) s.red[w] = x;
    __syncthreads();
    int base = 0, t = 0;
#pragma unroll
    for (int i = 0; i < kW; ++i) {
        const int r = s.red[i];
        base += i < w ? r : 0;
        t += r;
    }
    __syncthreads();
    total = t;
    return base + x - v;
}

// AND and OR of the nonzero keys, per wave, into s.wand / s.wor (read with
// and_or_read after a barrier): the bits every candidate shares need no
// radix pass.
template <class ForEach>
__device__ void and_or_publish(ForEach for_each, Shared &s)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t a = ~0u, o = 0u;
    bool zero = false;
    for_each([&](uint32_t key) {
        a &= key ? key : ~0u;
        o |= key;
        zero |= key == 0u;
    });
    a = wave_last(wave_scan_dpp(a, ~0u, [](uint32_t x, uint32_t y) { return x & y; }));
    o = wave_last(wave_scan_dpp(o, 0u, [](uint32_t x, uint32_t y) { return x | y; }));
    const bool wz = __builtin_amdgcn_ballot_w64(zero) != 0u;
    if (lane == 0) {
        s.wand[w] = a;
        s.wor[w] = o;
        s.wzero[w] = wz;
    }
}
// zero: some key of the workgroup is 0 (not a candidate)
__device__ __forceinline__ void and_or_read(const Shared &s, uint32_t &a, uint32_t &o, bool &zero)
{
    a = ~0u;
    o = 0u;
    uint32_t z = 0u;
#pragma unroll
    for (int i = 0; i < kW; ++i) {
        a &= s.wand[i];
        o |= s.wor[i];
        z |= s.wzero[i];
    }
    zero = z != 0u;
}
__device__ __forceinline__ void and_or_read(const Shared &s, uint32_t &a, uint32_t &o)
{
    bool zero;
    and_or_read(s, a, o, zero);
}

// Outcome of a radix select: keys with (key & M) > P are selected; of the
// cnt_eq keys with (key & M) == P, the rem with the lowest positions are.
// kk = min(k, number of nonzero keys) keys are selected in all.
struct Sel {
    uint32_t P, M;
    int rem, kk;
    int ceq;   // keys with (key & M) == P
};

// Wave 0, after a histogram pass: the bin d holding the rem-th largest key
// counted (rem = min(k, total) when k > 0: the first pass, which also
// reports the total), the keys in bins above d and in d.  Lane l sums bins
// 32l .. 32l+31 and one DPP scan over the lanes finds the lane L holding the
// bin; then lane j < 32 takes bin 32L + j and a second scan finds the bin,
// with no loop over bins.  The bins are cleared for the next pass.  Results
// in s.misc: d, keys above d, keys in d, total.
__device__ void find_bin(Shared &s, int rem, int k)
{
    const int lane = threadIdx.x & 63;
    uint32_t c[32];
    uint4 *h = (uint4 *)&s.hist[32 * lane];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint4 v = h[i];
        c[4 * i] = v.x;
        c[4 * i + 1] = v.y;
        c[4 * i + 2] = v.z;
        c[4 * i + 3] = v.w;
    }
#pragma unroll
    for (int st = 1; st < 32; st *= 2)
#pragma unroll
        for (int b = 0; b + st < 32; b += 2 * st) c[b] += c[b + st];
    const int sum = (int)c[0];
    const int incl = wave_incl_sum(sum);
    const int total = (int)wave_last((uint32_t)incl);
    if (k > 0) rem = min(k, total);
    const int above = total - incl;          // keys in bins past this lane's range
    const uint64_t hit = __builtin_amdgcn_ballot_w64(rem > 0 && above < rem && above + sum >= rem);
    int d = 0, A = 0, cd = 0;
    if (hit) {
        const int L = (int)__builtin_ctzll(hit);
        const int aL = __builtin_amdgcn_readlane(above, L);
        const int v = lane < 32 ? (int)s.hist[32 * L + lane] : 0;
        const int pre = wave_incl_sum(v);
        const int suf = __builtin_amdgcn_readlane(pre, 31) - pre + v;   // lane L's bins >= this one
        const uint64_t h2 = __builtin_amdgcn_ballot_w64(lane < 32 && aL + suf - v < rem && aL + suf >= rem);
        const int j = (int)__builtin_ctzll(h2);
        d = 32 * L + j;
        A = aL + __builtin_amdgcn_readlane(suf - v, j);
        cd = __builtin_amdgcn_readlane(v, j);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = make_uint4(0u, 0u, 0u, 0u);
    if (lane == 0) *(int4 *)s.misc = make_int4(d, A, cd, total);
}

// Radix select of the k largest nonzero keys.  for_each(f) calls f(key) for
// every key of the row; (a, o) = AND and OR of the nonzero keys (from
// and_or_publish).  Passes start below the bits every candidate shares and
// take 11 bits each, until the bin of the k-th key is taken whole.  The
// histogram bins are cleared by the caller before the first pass (and by
// find_bin after each).  With max_passes the select may stop early: then P
// (under M) is the prefix of the bin that holds the k-th key, so keys whose
// prefix is at least P include the k largest (a lower bound, not the cut).
template <class ForEach>
__device__ Sel radix_select(ForEach for_each, int k, uint32_t a, uint32_t o, Shared &s, bool nozero = false,
                           int max_passes = 32)
{
    const int tid = threadIdx.x;
    const uint32_t diff = a ^ o;
    int hb = diff ? 31 - __builtin_clz(diff) : 0;
    uint32_t M = ~((2u << hb) - 1u);          // hb == 31: 2u << 31 == 0, M == 0
    uint32_t P = a & M;
    int rem = 0, kk = 0, ceq = 0;
    bool first = true;
#pragma unroll 1
    for (;;) {
        const int lo = hb >= 10 ? hb - 10 : 0;
        const uint32_t dm = (2u << (hb - lo)) - 1u;
        if (first && nozero) {
            // every key is a candidate and shares the prefix of the AND/OR
            for_each([&](uint32_t key) { atomicAdd(&s.hist[(key >> lo) & dm], 1u); });
        } else {
            // only keys inside the prefix are counted: an LDS atomic costs per
            // active lane, and after the first pass few keys are inside
            for_each([&](uint32_t key) {
                if (key != 0u && (key & M) == P) atomicAdd(&s.hist[(key >> lo) & dm], 1u);
            });
        }
        __syncthreads();
        if (tid < kWave) find_bin(s, rem, first ? k : 0);
        __syncthreads();
        const int4 m4 = *(const int4 *)s.misc;
        if (first) {
            kk = min(k, m4.w);
            if (kk <= 0) return Sel{0u, 0u, 0, 0, 0};
            rem = kk;
            first = false;
        }
        rem -= m4.y;
        P |= (uint32_t)m4.x << lo;
        M |= dm << lo;
        if (m4.z == rem || lo == 0 || --max_passes == 0) {
            ceq = m4.z;
            break;
        }
        hb = lo - 1;
    }
    return Sel{P, M, rem, kk, ceq};
}

// every bin zero (before the first radix pass of a workgroup)
__device__ __forceinline__ void clear_hist(Shared &s)
{
    for (int i = (int)threadIdx.x; i < kBins; i += kT) s.hist[i] = 0u;
}

// Where the selected positions go.  IndexList: out[b][slot] = position.
// SparseIdx (the decode step's fused index build): the selection of token b
// becomes columns n_win + slot of its attention index row, each entry mapped
// to its compressed-pool row through the token's page table; the kernel also
// writes the window columns 0 .. n_win-1 (positions pos-n_win+1 .. pos).
struct IndexList {
    int32_t *out;
    __device__ IndexList(const TopkParams &p, int b) : out(p.out + (int64_t)b * p.out_sb) {}
    __device__ int value(int position) const { return position; }
    // values of a run of n consecutive positions from p0, prepared ahead
    struct Run {
        int p0;
    };
    __device__ Run run(int p0, int, int) const { return Run{p0}; }
    __device__ void run_rows(Run &) const {}
    __device__ int value_in(const Run &, int position) const { return position; }
    __device__ bool fast_run(const Run &) const { return true; }
    __device__ int value_fast(const Run &, int position) const { return position; }
    __device__ void put(int slot, int v) const { out[slot] = v; }
    __device__ void pad(int slot) const { out[slot] = -1; }
    struct Win {
    };
    __device__ Win window_begin() const { return Win{}; }
    __device__ void window_end(const Win &) const {}
    // no page table: the selected position is the output
    static constexpr int kStage = 1;
    struct Stage {
    };
    __device__ Stage stage_load(int) const { return Stage{}; }
    __device__ void stage_store(const Stage &, int32_t *, int) const {}
    __device__ int staged_value(int position, const int32_t *, int) const { return position; }
};
struct SparseIdx {
    int32_t *row;
    const int32_t *cmp_pt, *win_pt;
    int n_win, page, pos, sh;   // sh = log2(page) for power-of-two pages, else -1
    __device__ SparseIdx(const TopkParams &p, int b)
    {
        const int sq = p.seq[b];
        row = p.idx + (int64_t)b * p.idx_st;
        cmp_pt = p.cmp_pt + (int64_t)sq * p.cmp_pt_sb;
        win_pt = p.win_pt + (int64_t)sq * p.win_pt_sb;
        n_win = p.n_win;
        page = p.page;
        pos = p.pos[b];
        sh = (page & (page - 1)) == 0 ? 31 - __builtin_clz((uint32_t)page) : -1;
    }
    __device__ int value(int L) const
    {
        if (sh >= 0) return (cmp_pt[L >> sh] << sh) + (L & (page - 1));
        return cmp_pt[L / page] * page + L % page;
    }
    // a run of n <= page consecutive positions from p0 (below N) lies in the
    // page starting at base and the next one: their two page-table entries
    // are loaded up front, and no position needs a division
    // (b0, b1: the rows of the two pages' first entries, b1 less one page)
    struct Run {
        int base, n, b0, b1;
    };
    __device__ Run run(int p0, int n, int N) const
    {
        Run r{p0 - (sh >= 0 ? p0 & (page - 1) : p0 % page), n, 0, 0};
        if (p0 < N && n <= page) {
            const int last = min(p0 + n, N) - 1;
            r.b0 = cmp_pt[sh >= 0 ? p0 >> sh : p0 / page];
            r.b1 = cmp_pt[sh >= 0 ? last >> sh : last / page];
        }
        return r;
    }
    // the page-table entries have landed: their rows, once per run
    __device__ void run_rows(Run &r) const
    {
        r.b0 = sh >= 0 ? r.b0 << sh : r.b0 * page;
        r.b1 = (sh >= 0 ? r.b1 << sh : r.b1 * page) - page;
    }
    __device__ int value_in(const Run &r, int L) const
    {
        if (r.n > page) return value(L);   // pages shorter than a run: look each up
        return value_fast(r, L);
    }
    // the run lies in two pages whose entries are loaded: arithmetic only
    __device__ bool fast_run(const Run &r) const { return r.n <= page; }
    __device__ int value_fast(const Run &r, int L) const
    {
        const int off = L - r.base;
        return (off < page ? r.b0 : r.b1) + off;
    }
    __device__ void put(int slot, int v) const { row[n_win + slot] = v; }
    __device__ void pad(int slot) const { row[n_win + slot] = -1; }
    // window column j: row of position pos - (n_win - 1) + j, or -1
    __device__ int32_t window_row(int j) const
    {
        const int64_t q = (int64_t)pos - (n_win - 1) + j;
        if (q < 0) return -1;
        return sh >= 0 ? (win_pt[q >> sh] << sh) + (int32_t)(q & (page - 1))
                       : win_pt[q / page] * page + (int32_t)(q % page);
    }
    // the window columns: the page-table entry of column threadIdx.x loads
    // with the logits and is used after the selection.  The load is
    // unconditional (position clamped into 0 .. pos) so no branch around it
    // makes the wave wait for it before the logits go out.
    struct Win {
        int32_t e;
    };
    __device__ Win window_begin() const
    {
        if (pos < 0) return Win{0};
        const int64_t q = (int64_t)pos - (n_win - 1) + (int)threadIdx.x;
        const int64_t c = q < 0 ? 0 : (q > pos ? (int64_t)pos : q);
        return Win{win_pt[sh >= 0 ? c >> sh : c / page]};
    }
    __device__ void window_end(const Win &w) const
    {
        const int j = (int)threadIdx.x;
        if (j < n_win) {
            const int64_t q = (int64_t)pos - (n_win - 1) + j;
            row[j] = q < 0 ? -1
                           : (sh >= 0 ? (w.e << sh) + (int32_t)(q & (page - 1))
                                      : w.e * page + (int32_t)(q % page));
        }
        for (int jj = j + kT; jj < n_win; jj += kT) row[jj] = window_row(jj);
    }
    // The page-table entries of positions 0 .. N-1 go to LDS when they fit
    // (loaded with the logits, stored before the first barrier), so the
    // selected positions become rows without a memory round trip.
    static constexpr int kStage = 4096;
    static constexpr int kStagePT = kStage / kT;
    struct Stage {
        int32_t e[kStagePT];
    };
    __device__ int entries(int N) const
    {
        return N <= 0 ? 0 : (sh >= 0 ? ((N - 1) >> sh) + 1 : (N - 1) / page + 1);
    }
    __device__ Stage stage_load(int N) const
    {
        // no per-lane branch (indices clamped into the row) so the loads go
        // out together with the logits; rounds past the entries are skipped
        Stage st{};
        const int ne = entries(N);
        if (ne >= 1 && ne <= kStage) {
#pragma unroll
            for (int r = 0; r < kStagePT; ++r)
                if (r * kT < ne) st.e[r] = cmp_pt[min(r * kT + (int)threadIdx.x, ne - 1)];
        }
        return st;
    }
    __device__ void stage_store(const Stage &st, int32_t *ptab, int N) const
    {
        const int ne = entries(N);
        if (ne <= kStage) {
#pragma unroll
            for (int r = 0; r < kStagePT; ++r) {
                const int i = r * kT + (int)threadIdx.x;
                if (i < ne) ptab[i] = st.e[r];
            }
        }
    }
    __device__ int staged_value(int L, const int32_t *ptab, int N) const
    {
        const bool staged = entries(N) <= kStage;
        if (sh >= 0) return ((staged ? ptab[L >> sh] : cmp_pt[L >> sh]) << sh) + (L & (page - 1));
        return (staged ? ptab[L / page] : cmp_pt[L / page]) * page + L % page;
    }
};

// Places the selected positions of a block of KPT keys per thread in LDS by
// output slot, in position order: a selected key's slot is the number of
// greater keys before it plus min(equal keys before it, rem).  One scan of
// both counts (16 bits each) gives both.  gt_seen / eq_seen carry the counts
// of earlier blocks.  outv: LDS array of k slots plus kWave spare slots,
// where keys that are not selected write (so the unrolled loop below has no
// branches); flush_out writes the k slots out.  CHEAP: val_of is arithmetic,
// evaluated for every key; otherwise (it may load) only for selected ones.
template <int KPT, bool CHEAP, class ValOf>
__device__ void emit_block(const uint32_t (&key)[KPT], ValOf val_of, const Sel &q, int32_t *outv, int &gt_seen,
                           int &eq_seen, Shared &s)
{
    static_assert(KPT <= 32, "one bit per key");
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t gtm = 0u, eqm = 0u;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const uint32_t x = key[j] & q.M;
        gtm |= (x > q.P ? 1u : 0u) << j;
        eqm |= (x == q.P ? 1u : 0u) << j;
    }
    const int cnt = __builtin_popcount(gtm) | (__builtin_popcount(eqm) << 16);
    const int incl = wave_incl_sum(cnt);
    if (lane == 63) s.red[w] = incl;
    __syncthreads();
    int before = incl - cnt, tot = 0;
#pragma unroll
    for (int i = 0; i < kW; ++i) {
        const int r = s.red[i];
        before += i < w ? r : 0;
        tot += r;
    }
    const int g0 = gt_seen + (before & 0xFFFF), e0 = eq_seen + (before >> 16);
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const uint32_t below = (1u << j) - 1u;
        const int g = g0 + __builtin_popcount(gtm & below), e = e0 + __builtin_popcount(eqm & below);
        const bool gt = (gtm >> j) & 1u, eq = (eqm >> j) & 1u;
        const bool take = gt || (eq && e < q.rem);
        const int slot = take ? (gt ? g + min(e, q.rem) : g + e) : kMaxK + lane;
        if constexpr (CHEAP) {
            outv[slot] = val_of(j);
        } else {
            if (take) outv[slot] = val_of(j);
        }
    }
    gt_seen += tot & 0xFFFF;
    eq_seen += tot >> 16;
    __syncthreads();   // s.red is rewritten by the next block's scan
}

// Selection core in the strided layout: key[j] of thread t is entry j*kT + t
// of the row, so the 64 lanes of a wave hold consecutive entries and a
// ballot over one key column lists them in entry order.  A selected key's
// output slot is the number of selected keys before it: the selected keys of
// earlier (column, wave) pairs, from one exchange of per-pair counts, plus
// the lanes below it in its own ballot (mbcnt).

// Exclusive prefix of the per-(column j, wave w) counts in s.tab (entry
// j*kW + w, in entry order), for this wave's entry of every column.
template <int KPT>
__device__ void strided_bases(const int *tab, int (&base)[KPT])
{
    constexpr int R = KPT * kW / kWave;   // table entries per lane
    static_assert(R >= 1 && kW % R == 0, "KPT must be a multiple of 4");
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int v[R], sum = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        v[r] = tab[lane * R + r];
        sum += v[r];
    }
    const int incl = wave_incl_sum(sum);
    const int rr = w % R;
    int pre = incl - sum;
#pragma unroll
    for (int r = 0; r < R; ++r) pre += r < rr ? v[r] : 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) base[j] = __builtin_amdgcn_readlane(pre, j * (kW / R) + w / R);
}

__device__ __forceinline__ int rank_in(uint64_t m, int base)
{
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, (uint32_t)base));
}

// Writes the entry index of every selected key to outv[slot] (q.kk > 0, so
// P != 0 and keys of 0 are never selected); ends with a barrier.
template <int KPT>
__device__ void emit_strided(const uint32_t (&key)[KPT], const Sel &q, int32_t *outv, Shared &s)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, tid = threadIdx.x;
    int base[KPT];
    if (q.rem == q.ceq) {
        // the tie bin is taken whole: the selected keys are the keys >= P
        // (P has no bits below the mask)
        uint64_t m[KPT];
#pragma unroll
        for (int j = 0; j < KPT; ++j) m[j] = __builtin_amdgcn_ballot_w64(key[j] >= q.P);
        if (lane == 0) {
#pragma unroll
            for (int j = 0; j < KPT; ++j) s.tab[j * kW + w] = __builtin_popcountll(m[j]);
        }
        __syncthreads();
        strided_bases<KPT>(s.tab, base);
#pragma unroll
        for (int j = 0; j < KPT; ++j)
            if (key[j] >= q.P) outv[rank_in(m[j], base[j])] = j * kT + tid;
    } else {
        // keys of the tie bin are taken in entry order while fewer than rem
        // of them come before: slot = greater keys before + min(ties before, rem)
        uint64_t gm[KPT], em[KPT];
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const uint32_t x = key[j] & q.M;
            gm[j] = __builtin_amdgcn_ballot_w64(x > q.P);
            em[j] = __builtin_amdgcn_ballot_w64(x == q.P);
        }
        if (lane == 0) {
#pragma unroll
            for (int j = 0; j < KPT; ++j)
                s.tab[j * kW + w] = __builtin_popcountll(gm[j]) | (__builtin_popcountll(em[j]) << 16);
        }
        __syncthreads();
        strided_bases<KPT>(s.tab, base);
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const uint32_t x = key[j] & q.M;
            const int g = rank_in(gm[j], base[j] & 0xFFFF), e = rank_in(em[j], base[j] >> 16);
            if (x > q.P || (x == q.P && e < q.rem)) outv[g + min(e, q.rem)] = j * kT + tid;
        }
    }
    __syncthreads();
}

// the kk selected entry indices from LDS (placed by emit_strided), mapped to
// their outputs, then -1 up to k
template <class Out, class Map>
__device__ void flush_idx(const Out &out, int kk, int k, const int32_t *outv, Map map)
{
    for (int i = (int)threadIdx.x; i < k; i += kT) {
        if (i < kk) out.put(i, map(outv[i]));
        else out.pad(i);
    }
}

// the kk selected slots from LDS (placed by emit_block, which ends with a
// barrier), then -1 up to k, in coalesced stores
template <class Out>
__device__ void flush_out(const Out &out, int kk, int k, const int32_t *outv)
{
    for (int i = (int)threadIdx.x; i < k; i += kT) {
        if (i < kk) out.put(i, outv[i]);
        else out.pad(i);
    }
}

// KPT consecutive keys of positions base + tid*KPT .. from row x (n valid)
template <int KPT>
__device__ void load_keys(const float *x, int64_t base, int n, uint32_t (&key)[KPT])
{
    const int64_t p0 = base + (int64_t)threadIdx.x * KPT;
    const bool vec = ((reinterpret_cast<uintptr_t>(x) & 15u) == 0u) && (KPT % 4 == 0);
    if (vec && p0 + KPT <= n) {
#pragma unroll
        for (int j = 0; j < KPT; j += 4) {
            const float4 v = *(const float4 *)(x + p0 + j);
            key[j] = order_key(v.x);
            key[j + 1] = order_key(v.y);
            key[j + 2] = order_key(v.z);
            key[j + 3] = order_key(v.w);
        }
    } else {
#pragma unroll
        for (int j = 0; j < KPT; ++j) key[j] = p0 + j < n ? order_key(x[p0 + j]) : 0u;
    }
}

// the whole row streamed from memory: every pass reads it again
template <class Out>
__device__ void select_streaming(const float *x, int nv, int k, const Out &out, Shared &s, int32_t *outv)
{
    constexpr int KPT = 8;
    constexpr int BLK = kT * KPT;
    auto for_each = [&](auto f) {
        for (int base = 0; base < nv; base += BLK) {
            uint32_t key[KPT];
            load_keys<KPT>(x, base, nv, key);
#pragma unroll
            for (int j = 0; j < KPT; ++j) f(key[j]);
        }
    };
    clear_hist(s);
    and_or_publish(for_each, s);
    __syncthreads();
    uint32_t a, o;
    and_or_read(s, a, o);
    const Sel q = radix_select(for_each, k, a, o, s);
    const int kk = q.kk;
    int gt_seen = 0, eq_seen = 0;
    if (kk > 0) {
        for (int base = 0; base < nv; base += BLK) {
            uint32_t key[KPT];
            load_keys<KPT>(x, base, nv, key);
            const int p0 = base + (int)threadIdx.x * KPT;
            auto run = out.run(p0, KPT, nv);
            out.run_rows(run);
            if (out.fast_run(run))
                emit_block<KPT, true>(key, [&](int j) { return out.value_fast(run, p0 + j); }, q, outv, gt_seen,
                                      eq_seen, s);
            else
                emit_block<KPT, false>(key, [&](int j) { return out.value_in(run, p0 + j); }, q, outv, gt_seen,
                                       eq_seen, s);
        }
    }
    flush_out(out, kk, k, outv);
}

// rows of at most kT * KPT positions, keys in registers (strided layout)
template <int KPT, class Out>
__global__ __launch_bounds__(kT) void topk_direct_kernel(TopkParams p)
{
    __shared__ Shared s;
    __shared__ int32_t outv[kMaxK];             // selected entry indices by output slot
    __shared__ int32_t ptab[Out::kStage];       // page-table entries (fused index build)
    const int b = blockIdx.x, tid = threadIdx.x;
    const float *x = p.x + (int64_t)b * p.x_sb;
    const Out out(p, b);
    // the page-table entries, the window column, the count of valid entries
    // and the row's logits all load in one round trip
    const auto st = out.stage_load(p.N);
    const auto win = out.window_begin();
    const int nv_in = p.n_valid ? p.n_valid[b] : p.N;
    float v[KPT];
    if (p.N == KPT * kT) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) v[j] = x[j * kT + tid];
    } else if (p.N > 0) {
        // indices clamped into the row (no branch around the loads); entries
        // past N become -inf
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int i = j * kT + tid;
            const float t = x[min(i, p.N - 1)];
            v[j] = i < p.N ? t : -__builtin_inff();
        }
    } else {
#pragma unroll
        for (int j = 0; j < KPT; ++j) v[j] = -__builtin_inff();
    }
    uint32_t key[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) key[j] = order_key(v[j]);
    clear_hist(s);
    out.stage_store(st, ptab, p.N);
    const int nv = min(max(nv_in, 0), p.N);
    if (nv < p.N) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) key[j] = j * kT + tid < nv ? key[j] : 0u;
    }
    auto for_each = [&](auto f) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) f(key[j]);
    };
    and_or_publish(for_each, s);
    __syncthreads();
    uint32_t a, o;
    bool zero;
    and_or_read(s, a, o, zero);
    const Sel q = radix_select(for_each, p.k, a, o, s, !zero);
    if (q.kk > 0) emit_strided<KPT>(key, q, outv, s);
    out.window_end(win);
    flush_idx(out, q.kk, p.k, outv, [&](int i) { return out.staged_value(i, ptab, p.N); });
}

// workspace of the two-launch path, per row: chunk counts, the sample
// threshold, and per chunk kSlotCap keys and positions
struct TopkWs {
    int *count;        // [B][nch]
    uint32_t *tau;     // [B]
    uint32_t *key;     // [B][nch][kSlotCap]
    int32_t *pos;      // [B][nch][kSlotCap]
};

__host__ __device__ inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

__host__ __device__ inline TopkWs topk_ws(void *base, int B, int nch)
{
    uint8_t *p = (uint8_t *)base;
    TopkWs w;
    w.count = (int *)p;
    p += align256((size_t)B * nch * 4);
    w.tau = (uint32_t *)p;
    p += align256((size_t)B * 4);
    w.key = (uint32_t *)p;
    p += align256((size_t)B * nch * kSlotCap * 4);
    w.pos = (int32_t *)p;
    return w;
}

__host__ __device__ inline size_t topk_ws_size(int B, int nch)
{
    return align256((size_t)B * nch * 4) + align256((size_t)B * 4) + 2 * align256((size_t)B * nch * kSlotCap * 4);
}

// filter launch: grid (chunks, B)
__global__ __launch_bounds__(kT) void topk_filter_kernel(TopkParams p, int nch)
{
    __shared__ Shared s;
    const int c = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const float *x = p.x + (int64_t)b * p.x_sb;
    int nv = p.n_valid ? p.n_valid[b] : p.N;
    nv = min(max(nv, 0), p.N);
    const TopkWs ws = topk_ws(p.workspace, p.B, nch);

    // this chunk's keys load together with the sample below (one memory
    // round trip for both)
    constexpr int KPT = kChunk / kT;
    uint32_t key[KPT];
    const int64_t base = (int64_t)c * kChunk;
    load_keys<KPT>(x, base, nv, key);

    // threshold from the fixed strided sample (identical in every chunk)
    uint32_t tau = 1u;
    if (nv > kSample) {
        clear_hist(s);   // ordered before the first radix pass by the scan's barriers
        constexpr int SPT = kSample / kT;
        uint32_t sk[SPT];
#pragma unroll
        for (int j = 0; j < SPT; ++j) sk[j] = order_key(x[(int64_t)(tid * SPT + j) * nv / kSample]);
        int nz = 0;
#pragma unroll
        for (int j = 0; j < SPT; ++j) nz += sk[j] != 0u;
        auto for_each = [&](auto f) {
#pragma unroll
            for (int j = 0; j < SPT; ++j) f(sk[j]);
        };
        and_or_publish(for_each, s);   // read after the scan's barriers
        int ns;
        block_excl_scan(nz, s, ns);
        const int want = min(kSample, (int)(((int64_t)2 * p.k * kSample + nv - 1) / nv) + 16);
        if (ns >= want) {
            uint32_t a, o;
            and_or_read(s, a, o);
            // one pass: the bin of the want-th sample key bounds the cut from
            // below (the select launch is exact whatever tau admits, and
            // falls back to a streamed select when fewer than k pass)
            tau = radix_select(for_each, want, a, o, s, false, 1).P;   // low bits zero: key >= tau <=> prefix >= P
            if (tau == 0u) tau = 1u;
        }
    }
    if (c == 0 && tid == 0) ws.tau[b] = tau;

    int n = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        key[j] = key[j] >= tau ? key[j] : 0u;
        n += key[j] != 0u;
    }
    int total;
    int o = block_excl_scan(n, s, total);
    const size_t slot = ((size_t)b * nch + c) * kSlotCap;
    if (total <= kSlotCap) {
#pragma unroll
        for (int j = 0; j < KPT; ++j)
            if (key[j]) {
                ws.key[slot + o] = key[j];
                ws.pos[slot + o] = (int32_t)(base + tid * KPT + j);
                ++o;
            }
    }
    if (tid == 0) ws.count[(size_t)b * nch + c] = total;
}

// select launch: grid (B)
template <class Out>
__global__ __launch_bounds__(kT) void topk_select_kernel(TopkParams p, int nch)
{
    constexpr int KPT = kDirectMax / kT;
    __shared__ Shared s;
    __shared__ uint32_t ckey[kDirectMax];
    __shared__ int32_t cpos[kDirectMax];
    __shared__ int offs[kMaxChunks];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const float *x = p.x + (int64_t)b * p.x_sb;
    const Out out(p, b);
    const auto win = out.window_begin();
    int nv = p.n_valid ? p.n_valid[b] : p.N;
    nv = min(max(nv, 0), p.N);
    const TopkWs ws = topk_ws(p.workspace, p.B, nch);
    const int *cnt = ws.count + (size_t)b * nch;

    // The first 64 entries of this wave's first SPC chunks load together
    // with the counts (a slot holds kSlotCap >= 64 entries, so the reads stay
    // inside it; entries past a chunk's count are never used).
    constexpr int SPC = 4;
    uint32_t sk[SPC];
    int32_t sp[SPC];
#pragma unroll
    for (int r = 0; r < SPC; ++r) {
        const int ci = w + r * kW;
        sk[r] = 0u;
        sp[r] = 0;
        if (ci < nch) {
            const size_t slot = ((size_t)b * nch + ci) * kSlotCap + lane;
            sk[r] = ws.key[slot];
            sp[r] = ws.pos[slot];
        }
    }

    // slot offsets in chunk (= position) order, in one scan: a chunk whose
    // slot overflowed counts kDirectMax + 1, which sends the row to the
    // streaming path (total < 2^27: kMaxChunks chunks of at most that)
    constexpr int CPT = kMaxChunks / kT;
    int cl[CPT], local = 0;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int ci = tid * CPT + j;
        const int c = ci < nch ? cnt[ci] : 0;
        cl[j] = c > kSlotCap ? kDirectMax + 1 : c;
        local += cl[j];
    }
    int total;
    int o = block_excl_scan(local, s, total);
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int ci = tid * CPT + j;
        if (ci < nch) offs[ci] = o;
        o += cl[j];
    }
    const uint32_t tau = ws.tau[b];
    clear_hist(s);   // ordered before the first radix pass by the barriers below
    const bool ok = total <= kDirectMax && (total >= p.k || tau == 1u);
    // the selection by output slot reuses ckey: it is read into registers
    // before the first barrier of the radix select
    int32_t *const outv = (int32_t *)ckey;
    if (!ok) {
        select_streaming(x, nv, p.k, out, s, outv);
        out.window_end(win);
        return;
    }
    __syncthreads();
    // gather the slots into LDS, one wave per chunk; a chunk's count is the
    // difference of its offsets
    auto gather_chunk = [&](int ci, int from) __attribute__((always_inline)) {
        const int at = offs[ci], n = (ci + 1 < nch ? offs[ci + 1] : total) - at;
        const size_t slot = ((size_t)b * nch + ci) * kSlotCap;
        for (int i = from + lane; i < n; i += kWave) {
            ckey[at + i] = ws.key[slot + i];
            cpos[at + i] = ws.pos[slot + i];
        }
        return n;
    };
#pragma unroll
    for (int r = 0; r < SPC; ++r) {
        const int ci = w + r * kW;
        if (ci < nch) {
            const int n = gather_chunk(ci, kWave);   // entries past the first 64
            if (lane < n) {
                ckey[offs[ci] + lane] = sk[r];
                cpos[offs[ci] + lane] = sp[r];
            }
        }
    }
    for (int ci = w + SPC * kW; ci < nch; ci += kW) gather_chunk(ci, 0);
    __syncthreads();
    const int kk = min(p.k, total);
    // candidates in registers (strided layout): 8 per thread when they fit
    // (the usual case), else 16; every candidate is nonzero
    auto select_core = [&](auto kpt_tag) __attribute__((always_inline)) {
        constexpr int K = decltype(kpt_tag)::value;
        uint32_t key[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const int i = j * kT + tid;
            key[j] = i < total ? ckey[i] : 0u;
        }
        if (kk > 0) {
            auto for_each = [&](auto f) {
#pragma unroll
                for (int j = 0; j < K; ++j) f(key[j]);
            };
            and_or_publish(for_each, s);
            __syncthreads();
            uint32_t a, o;
            bool zero;
            and_or_read(s, a, o, zero);
            const Sel q = radix_select(for_each, kk, a, o, s, !zero);
            emit_strided<K>(key, q, outv, s);
        }
    };
    if (total <= 8 * kT) select_core(std::integral_constant<int, 8>{});
    else select_core(std::integral_constant<int, KPT>{});
    out.window_end(win);
    flush_idx(out, kk, p.k, outv, [&](int i) { return out.value(cpos[i]); });
}

template <class Out>
__global__ __launch_bounds__(kT) void topk_stream_kernel(TopkParams p)
{
    __shared__ Shared s;
    __shared__ int32_t outv[kMaxK + kWave];   // the selection by output slot, then spare slots
    const int b = blockIdx.x;
    int nv = p.n_valid ? p.n_valid[b] : p.N;
    nv = min(max(nv, 0), p.N);
    const Out out(p, b);
    const auto win = out.window_begin();
    select_streaming(p.x + (int64_t)b * p.x_sb, nv, p.k, out, s, outv);
    out.window_end(win);
}

int n_chunks(int N) { return (N + kChunk - 1) / kChunk; }

}  // namespace

size_t topk_workspace_bytes(int B, int N, int k)
{
    (void)k;
    if (N <= kDirectMax || n_chunks(N) > kMaxChunks) return 0;
    return topk_ws_size(B, n_chunks(N));
}

namespace {

template <class Out>
hipError_t launch_topk_t(const TopkParams &p, hipStream_t st)
{
    if (p.B == 0) return hipSuccess;
    if (p.N <= kDirectMax) {
        static_assert(kDirectMax == kMaxKPT * kT, "direct rows fit the largest core");
        if (p.N <= 8 * kT) hipLaunchKernelGGL((topk_direct_kernel<8, Out>), dim3((unsigned)p.B), dim3(kT), 0, st, p);
        else hipLaunchKernelGGL((topk_direct_kernel<kMaxKPT, Out>), dim3((unsigned)p.B), dim3(kT), 0, st, p);
        return hipGetLastError();
    }
    const int nch = n_chunks(p.N);
    if (nch > kMaxChunks) {
        hipLaunchKernelGGL((topk_stream_kernel<Out>), dim3((unsigned)p.B), dim3(kT), 0, st, p);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(topk_filter_kernel, dim3((unsigned)nch, (unsigned)p.B), dim3(kT), 0, st, p, nch);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((topk_select_kernel<Out>), dim3((unsigned)p.B), dim3(kT), 0, st, p, nch);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const TopkParams &p, hipStream_t st)
{
    return p.idx ? launch_topk_t<SparseIdx>(p, st) : launch_topk_t<IndexList>(p, st);
}

}  // namespace sap
