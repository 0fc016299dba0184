// Client-side top-k selection for partial sharing, for gfx950.
//
// A client shares only the fraction of its update it chooses ("NVIDIA Clara
// implements federated learning", epnc.co.kr, introduction and client-side
// workflow section); it keeps the k = floor(p*N) entries of largest
// magnitude.  Order: by the magnitude bit pattern (the fp32 bits with the sign
// cleared; bf16 values widened to fp32 exactly), which is |value| order with
// NaNs above infinity and -0 tied with +0; ties go to the lower index.  The
// output is the k chosen indices in increasing order, with their values as
// fp32 -- the (index, value) list the sparse merge takes.
//
// Exact radix select over the 31-bit key, most significant digit first
// (11, 11, 9 bits; bf16 keys have 15 bits and need only the first two digits):
// each pass histograms, in LDS, the keys that agree with the digits chosen so
// far, and a one-workgroup step picks the digit holding the k-th largest key.
// After the last digit the threshold key T is exact, together with r, the
// number of keys equal to T that are kept (the r lowest-indexed ones).  Then
// per tile of TK_TILE elements: counts of keys > T and == T; one workgroup
// scans those counts into each tile's output offset and share of the r ties;
// and each tile writes its chosen entries in index order.  Every pass is a
// plain stream over the input (HBM-bound); no workgroup ever waits on
// another.
#include <hip/hip_runtime.h>

#include "fedavg_internal.h"

namespace fa {

namespace {

constexpr int TK_THREADS = 256;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int TK_MAX_BINS = 2048;

using u32x4 = __attribute__((ext_vector_type(4))) unsigned int;

struct TopkState {
    uint32_t prefix; // key bits chosen so far (the threshold key T at the end)
    uint32_t pad;
    int64_t rank;    // how many keys matching `prefix` are still to be kept
};

__device__ __forceinline__ uint32_t key_f32(uint32_t bits) { return bits & 0x7FFFFFFFu; }
__device__ __forceinline__ uint32_t key_bf16(uint32_t bits16) { return (bits16 << 16) & 0x7FFFFFFFu; }

// Element e's key and fp32 value.
template <int DT> __device__ __forceinline__ uint32_t key_at(const void *x, int64_t e)
{
    if constexpr (DT == DT_F32)
        return key_f32(static_cast<const uint32_t *>(x)[e]);
    else
        return key_bf16(static_cast<const uint16_t *>(x)[e]);
}

template <int DT> __device__ __forceinline__ float value_at(const void *x, int64_t e)
{
    if constexpr (DT == DT_F32)
        return static_cast<const float *>(x)[e];
    else
        return __uint_as_float((uint32_t) static_cast<const uint16_t *>(x)[e] << 16);
}

// Keys of one 16-byte vector: 4 fp32 or 8 bf16 values.
template <int DT> struct Vec;
template <> struct Vec<DT_F32> {
    static constexpr int N = 4;
    __device__ static void keys(const void *x, int64_t v, uint32_t k[N])
    {
        const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(x) + v);
        k[0] = key_f32(r.x);
        k[1] = key_f32(r.y);
        k[2] = key_f32(r.z);
        k[3] = key_f32(r.w);
    }
};
template <> struct Vec<DT_BF16> {
    static constexpr int N = 8;
    __device__ static void keys(const void *x, int64_t v, uint32_t k[N])
    {
        const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(x) + v);
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            k[2 * j] = key_bf16(w[j] & 0xFFFFu);
            k[2 * j + 1] = key_bf16(w[j] >> 16);
        }
    }
};

__global__ void topk_init_kernel(unsigned long long *hist, TopkState *st, int64_t k)
{
    for (int b = threadIdx.x; b < TK_MAX_BINS; b += blockDim.x)
        hist[b] = 0ull;
    if (threadIdx.x == 0) {
        st->prefix = 0u;
        st->pad = 0u;
        st->rank = k;
    }
}

// Histogram of digit (key >> shift) & (bins-1) over the keys whose bits above
// the digit equal the prefix chosen so far.  One LDS histogram per wave keeps
// the waves off each other's counters; a workgroup adds its totals to the
// global histogram once.
template <int DT>
__global__ __launch_bounds__(TK_THREADS) void topk_hist_kernel(const void *x, int64_t N,
                                                               bool vec_ok,
                                                               unsigned long long *hist,
                                                               const TopkState *st, int shift,
                                                               int bits)
{
    __shared__ uint32_t s_hist[TK_WAVES][TK_MAX_BINS];
    const int bins = 1 << bits;
    const uint32_t above = (shift + bits >= 31) ? 0u : (0x7FFFFFFFu >> (shift + bits)) << (shift + bits);
    const uint32_t prefix = st->prefix & above;
    const int wave = threadIdx.x >> 6;
    for (int b = threadIdx.x; b < TK_WAVES * bins; b += blockDim.x)
        s_hist[b / bins][b % bins] = 0u;
    __syncthreads();

    uint32_t *h = s_hist[wave];
    constexpr int V = Vec<DT>::N;
    const int64_t nvec = vec_ok ? N / V : 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
        uint32_t k[V];
        Vec<DT>::keys(x, v, k);
#pragma unroll
        for (int j = 0; j < V; ++j)
            if ((k[j] & above) == prefix)
                atomicAdd(&h[(k[j] >> shift) & (uint32_t)(bins - 1)], 1u);
    }
    for (int64_t e = nvec * V + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < N; e += stride) {
        const uint32_t k = key_at<DT>(x, e);
        if ((k & above) == prefix)
            atomicAdd(&h[(k >> shift) & (uint32_t)(bins - 1)], 1u);
    }
    __syncthreads();
    for (int b = threadIdx.x; b < bins; b += blockDim.x) {
        uint32_t c = 0;
#pragma unroll
        for (int w = 0; w < TK_WAVES; ++w)
            c += s_hist[w][b];
        if (c)
            atomicAdd(&hist[b], (unsigned long long)c);
    }
}

// One workgroup of TK_SELECT_THREADS: the largest digit d with
// sum_{u >= d} hist[u] >= rank joins the prefix, rank drops by the count of
// larger digits, and the histogram is cleared for the next pass.
constexpr int TK_SELECT_THREADS = 1024;

__global__ __launch_bounds__(TK_SELECT_THREADS) void topk_select_kernel(unsigned long long *hist,
                                                                        TopkState *st, int shift,
                                                                        int bits)
{
    __shared__ unsigned long long s_suffix[TK_MAX_BINS + 1];
    const int bins = 1 << bits;
    const int t = threadIdx.x;
    // read before the first barrier: one thread rewrites it at the end
    const int64_t rank = st->rank;
    for (int b = t; b < bins; b += blockDim.x)
        s_suffix[b] = hist[b];
    if (t == 0)
        s_suffix[bins] = 0ull;
    __syncthreads();
    // suffix sums, bin by bin from the top: a Hillis-Steele scan over at most
    // 2048 entries, each step reading before any thread writes
    for (int d = 1; d < bins; d <<= 1) {
        unsigned long long add[2] = {0ull, 0ull};
        for (int i = 0, b = t; b < bins; b += blockDim.x, ++i)
            add[i] = b + d < bins ? s_suffix[b + d] : 0ull;
        __syncthreads();
        for (int i = 0, b = t; b < bins; b += blockDim.x, ++i)
            s_suffix[b] += add[i];
        __syncthreads();
    }
    for (int b = t; b < bins; b += blockDim.x) {
        if ((int64_t)s_suffix[b] >= rank && (int64_t)s_suffix[b + 1] < rank) {
            st->prefix |= (uint32_t)b << shift;
            st->rank = rank - (int64_t)s_suffix[b + 1];
        }
    }
    for (int b = t; b < TK_MAX_BINS; b += blockDim.x)
        hist[b] = 0ull;
}

// Per tile: how many keys exceed the threshold and how many equal it.
template <int DT>
__global__ __launch_bounds__(TK_THREADS) void topk_count_kernel(const void *x, int64_t N,
                                                                bool vec_ok, const TopkState *st,
                                                                uint32_t *gt, uint32_t *eq)
{
    __shared__ uint32_t s_sum[TK_WAVES];
    constexpr int V = Vec<DT>::N;
    constexpr int ROUNDS = TK_TILE / (TK_THREADS * V);
    const uint32_t T = st->prefix;
    const int64_t tile0 = (int64_t)blockIdx.x * TK_TILE;
    uint32_t ngt = 0, neq = 0;
    if (vec_ok && tile0 + TK_TILE <= N) {
#pragma unroll
        for (int j = 0; j < ROUNDS; ++j) {
            uint32_t k[V];
            Vec<DT>::keys(x, (tile0 + (int64_t)(j * TK_THREADS + threadIdx.x) * V) / V, k);
#pragma unroll
            for (int q = 0; q < V; ++q) {
                ngt += k[q] > T;
                neq += k[q] == T;
            }
        }
    } else {
        const int64_t end = min(tile0 + (int64_t)TK_TILE, N);
        for (int64_t e = tile0 + threadIdx.x; e < end; e += TK_THREADS) {
            const uint32_t k = key_at<DT>(x, e);
            ngt += k > T;
            neq += k == T;
        }
    }
    // packed: both counts stay below 2^16 within a tile
    uint32_t c = (ngt << 16) | neq;
    for (int off = 32; off > 0; off >>= 1)
        c += __shfl_down(c, off, 64);
    if ((threadIdx.x & 63) == 0)
        s_sum[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t s = 0;
        for (int w = 0; w < TK_WAVES; ++w)
            s += s_sum[w];
        gt[blockIdx.x] = s >> 16;
        eq[blockIdx.x] = s & 0xFFFFu;
    }
}

// Exclusive scan helper for one workgroup of TK_SELECT_THREADS threads over
// per-thread totals; returns the thread's exclusive prefix and the grand
// total through `total`.
__device__ int64_t block_exclusive_scan(int64_t v, int64_t *s_tmp, int64_t &total)
{
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    int64_t inc = v;
    for (int off = 1; off < 64; off <<= 1) {
        const int64_t o = __shfl_up(inc, off, 64);
        if (lane >= off)
            inc += o;
    }
    if (lane == 63)
        s_tmp[wave] = inc;
    __syncthreads();
    if (t == 0) {
        int64_t run = 0;
        for (int w = 0; w < TK_SELECT_THREADS / 64; ++w) {
            const int64_t x = s_tmp[w];
            s_tmp[w] = run;
            run += x;
        }
        s_tmp[TK_SELECT_THREADS / 64] = run;
    }
    __syncthreads();
    const int64_t ex = s_tmp[wave] + inc - v;
    total = s_tmp[TK_SELECT_THREADS / 64];
    __syncthreads();
    return ex;
}

// One workgroup: tile b keeps take[b] = clamp(r - (ties before b), 0, eq[b])
// of its ties, and writes from off[b] = sum over earlier tiles of
// gt + take.  Each thread owns a contiguous run of tiles.
__global__ __launch_bounds__(TK_SELECT_THREADS) void topk_scan_kernel(int64_t nt, const TopkState *st,
                                                                      const uint32_t *gt,
                                                                      const uint32_t *eq,
                                                                      uint32_t *take, int64_t *off)
{
    __shared__ int64_t s_tmp[TK_SELECT_THREADS / 64 + 1];
    const int64_t per = (nt + TK_SELECT_THREADS - 1) / TK_SELECT_THREADS;
    const int64_t b0 = min((int64_t)threadIdx.x * per, nt), b1 = min(b0 + per, nt);
    const int64_t r = st->rank;
    int64_t total;
    int64_t my = 0;
    for (int64_t b = b0; b < b1; ++b)
        my += eq[b];
    int64_t ties_before = block_exclusive_scan(my, s_tmp, total);
    int64_t sel = 0;
    for (int64_t b = b0; b < b1; ++b) {
        const int64_t tk = max((int64_t)0, min(r - ties_before, (int64_t)eq[b]));
        take[b] = (uint32_t)tk;
        ties_before += eq[b];
        sel += gt[b] + tk;
    }
    int64_t run = block_exclusive_scan(sel, s_tmp, total);
    for (int64_t b = b0; b < b1; ++b) {
        off[b] = run;
        run += gt[b] + take[b];
    }
}

// Per tile: write the kept entries in index order.  Round j of the tile has
// thread t holding V consecutive elements; one workgroup scan per round of the
// packed (above, tie) counts gives every element its rank among the tile's
// kept entries.
template <int DT>
__global__ __launch_bounds__(TK_THREADS) void topk_write_kernel(const void *x, int64_t N,
                                                                bool vec_ok, const TopkState *st,
                                                                const uint32_t *take,
                                                                const int64_t *off, int64_t k_out,
                                                                int64_t *idx_out, float *val_out)
{
    __shared__ uint32_t s_wave[TK_WAVES + 1];
    constexpr int V = Vec<DT>::N;
    constexpr int ROUNDS = TK_TILE / (TK_THREADS * V);
    const uint32_t T = st->prefix;
    const int64_t tile0 = (int64_t)blockIdx.x * TK_TILE;
    const uint32_t tk = take[blockIdx.x];
    const int64_t base = off[blockIdx.x];
    const bool full = vec_ok && tile0 + TK_TILE <= N;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t carry_gt = 0, carry_eq = 0; // counts in the rounds before this one
    for (int j = 0; j < ROUNDS; ++j) {
        const int64_t e0 = tile0 + (int64_t)(j * TK_THREADS + threadIdx.x) * V;
        uint32_t k[V];
        if (full) {
            Vec<DT>::keys(x, e0 / V, k);
        } else {
#pragma unroll
            for (int q = 0; q < V; ++q)
                k[q] = e0 + q < N ? key_at<DT>(x, e0 + q) : 0u;
        }
        uint32_t ngt = 0, neq = 0;
#pragma unroll
        for (int q = 0; q < V; ++q) {
            const bool in = full || e0 + q < N;
            ngt += in && k[q] > T;
            neq += in && k[q] == T;
        }
        // inclusive wave scan of the packed counts, then across the waves
        const uint32_t c = (ngt << 16) | neq;
        uint32_t inc = c;
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t o = __shfl_up(inc, d, 64);
            if (lane >= d)
                inc += o;
        }
        if (lane == 63)
            s_wave[wave] = inc;
        __syncthreads();
        uint32_t before = 0, round_total = 0;
        for (int w = 0; w < TK_WAVES; ++w) {
            const uint32_t s = s_wave[w];
            before += w < wave ? s : 0u;
            round_total += s;
        }
        __syncthreads(); // s_wave is rewritten next round
        const uint32_t ex = before + inc - c;
        uint32_t gt_before = carry_gt + (ex >> 16);
        uint32_t eq_before = carry_eq + (ex & 0xFFFFu);
        carry_gt += round_total >> 16;
        carry_eq += round_total & 0xFFFFu;
        if (ngt + neq == 0)
            continue;
#pragma unroll
        for (int q = 0; q < V; ++q) {
            const bool in = full || e0 + q < N;
            if (!in)
                continue;
            // positions stay below k when the counts are consistent; the
            // bound keeps any inconsistency from writing out of range
            if (k[q] > T) {
                const int64_t pos = base + gt_before + min(eq_before, tk);
                if (pos < k_out) {
                    idx_out[pos] = e0 + q;
                    val_out[pos] = value_at<DT>(x, e0 + q);
                }
                ++gt_before;
            } else if (k[q] == T) {
                if (eq_before < tk) {
                    const int64_t pos = base + gt_before + eq_before;
                    if (pos < k_out) {
                        idx_out[pos] = e0 + q;
                        val_out[pos] = value_at<DT>(x, e0 + q);
                    }
                }
                ++eq_before;
            }
        }
    }
}

unsigned grid_of(int64_t work, int64_t cap)
{
    int64_t g = (work + TK_THREADS - 1) / TK_THREADS;
    if (g > cap)
        g = cap;
    return (unsigned)(g < 1 ? 1 : g);
}

template <int DT>
hipError_t topk_run(const void *x, int64_t N, int64_t k, int64_t *idx_out, float *val_out,
                    void *ws, int cus, hipStream_t s)
{
    char *w = static_cast<char *>(ws);
    auto *hist = reinterpret_cast<unsigned long long *>(w);
    auto *st = reinterpret_cast<TopkState *>(w + TK_MAX_BINS * 8);
    const int64_t nt = (N + TK_TILE - 1) / TK_TILE;
    char *tiles = w + TK_MAX_BINS * 8 + 256;
    auto *off = reinterpret_cast<int64_t *>(tiles);
    auto *gt = reinterpret_cast<uint32_t *>(tiles + nt * 8);
    auto *eq = gt + nt;
    auto *take = eq + nt;
    const bool vec_ok = (reinterpret_cast<uintptr_t>(x) & 15u) == 0;

    topk_init_kernel<<<1, 256, 0, s>>>(hist, st, k);
    // digits of the 31-bit key: bits 30..20, 19..9, 8..0 (bf16 keys end at bit 16)
    const int shifts[3] = {20, 9, 0};
    const int widths[3] = {11, 11, 9};
    const int passes = DT == DT_F32 ? 3 : 2;
    const unsigned hg = grid_of(N / Vec<DT>::N + 1, (int64_t)cus * 4);
    for (int p = 0; p < passes; ++p) {
        topk_hist_kernel<DT><<<hg, TK_THREADS, 0, s>>>(x, N, vec_ok, hist, st, shifts[p], widths[p]);
        topk_select_kernel<<<1, TK_SELECT_THREADS, 0, s>>>(hist, st, shifts[p], widths[p]);
    }
    topk_count_kernel<DT><<<(unsigned)nt, TK_THREADS, 0, s>>>(x, N, vec_ok, st, gt, eq);
    topk_scan_kernel<<<1, TK_SELECT_THREADS, 0, s>>>(nt, st, gt, eq, take, off);
    topk_write_kernel<DT><<<(unsigned)nt, TK_THREADS, 0, s>>>(x, N, vec_ok, st, take, off, k,
                                                              idx_out, val_out);
    return hipGetLastError();
}

} // namespace

size_t topk_workspace_bytes(int64_t N)
{
    const int64_t nt = (N + TK_TILE - 1) / TK_TILE;
    return (size_t)TK_MAX_BINS * 8 + 256 + (size_t)nt * (8 + 4 + 4 + 4);
}

hipError_t launch_topk(const void *x, int dt, int64_t N, int64_t k, int64_t *idx_out,
                       float *val_out, void *ws, int cus, hipStream_t s)
{
    return dt == DT_F32 ? topk_run<DT_F32>(x, N, k, idx_out, val_out, ws, cus, s)
                        : topk_run<DT_BF16>(x, N, k, idx_out, val_out, ws, cus, s);
}

} // namespace fa
