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
// Exact radix select over the 31-bit key, most significant digit first, in
// digits of 11, 11 and 9 bits (bf16 keys have 15 bits: two digits decide
// them).  Three passes read the whole input:
//   1. a histogram of the top digit (LDS histograms, one global add per bin
//      and workgroup), after which one workgroup picks the digit b1 that
//      holds the k-th largest key;
//   2. per tile of TK_TILE elements: the keys above bin b1 are counted, and
//      the keys inside it -- the candidates, a few per cent of the input for
//      smooth data -- are compacted into a buffer as (key, position in tile);
//   3. after the remaining digits are chosen from histograms of the
//      candidates only, and each tile's counts of keys above and equal to the
//      threshold T come from its candidates, one workgroup scans the counts
//      into output offsets and each tile's share of the ties (the lowest
//      indices), and each tile writes its kept entries in index order.
// If the candidates outgrow their buffer (heavily tied data), a flag in the
// workspace sends every later kernel down the same steps over the whole
// input instead; the result is the same.  No workgroup ever waits on
// another.
#include <hip/hip_runtime.h>

#include "fedavg_internal.h"

namespace fa {

namespace {

constexpr int TK_THREADS = 256; // histogram kernels
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int TT_THREADS = 256; // per-tile kernels
constexpr int TT_WAVES = TT_THREADS / 64;
constexpr int TK_MAX_BINS = 2048;
constexpr int TK_SELECT_THREADS = 1024;
constexpr int TK_TOP_SHIFT = 20; // first digit: key bits 30..20

using u32x2 = __attribute__((ext_vector_type(2))) unsigned int;
using u32x4 = __attribute__((ext_vector_type(4))) unsigned int;

constexpr int TK_REGIONS = 256; // candidate regions, each with its own counter

struct TopkState {
    uint32_t prefix;             // key bits chosen so far (the threshold T at the end)
    uint32_t overflow;           // candidates did not fit: use the whole input
    int64_t rank;                // keys matching `prefix` still to be kept
};

// Where the pieces of the workspace live.
struct TopkWs {
    unsigned long long *hist;
    TopkState *st;
    int64_t *off;        // per tile: first output position
    uint32_t *gt, *eq;   // per tile: keys above / equal to T
    uint32_t *take;      // per tile: ties kept
    uint32_t *def;       // per tile: keys above bin b1
    uint32_t *ccnt;      // per tile: candidates
    unsigned long long *coff; // per tile: first candidate
    u32x2 *cand;         // (key, position in tile), TK_REGIONS regions of rcap
    unsigned long long *rcount; // per region: candidates reserved
    int64_t rcap;        // candidates per region
};

__host__ __device__ constexpr int64_t round4(int64_t n) { return (n + 3) / 4 * 4; }

// Candidates per region: the regions together hold N/16 + 64Ki entries.
int64_t region_capacity(int64_t N) { return (N / 16 + 65536 + TK_REGIONS - 1) / TK_REGIONS; }

TopkWs carve(void *ws, int64_t N)
{
    const int64_t nt = (N + TK_TILE - 1) / TK_TILE;
    const int64_t ntp = round4(nt);
    char *w = static_cast<char *>(ws);
    TopkWs p;
    p.hist = reinterpret_cast<unsigned long long *>(w);
    w += TK_MAX_BINS * 8;
    p.st = reinterpret_cast<TopkState *>(w);
    w += 256;
    p.rcount = reinterpret_cast<unsigned long long *>(w);
    w += TK_REGIONS * 8;
    p.off = reinterpret_cast<int64_t *>(w);
    w += ntp * 8;
    p.coff = reinterpret_cast<unsigned long long *>(w);
    w += ntp * 8;
    p.gt = reinterpret_cast<uint32_t *>(w);
    p.eq = p.gt + ntp;
    p.take = p.eq + ntp;
    p.def = p.take + ntp;
    p.ccnt = p.def + ntp;
    w += ntp * 4 * 5;
    p.cand = reinterpret_cast<u32x2 *>(w);
    p.rcap = region_capacity(N);
    return p;
}

__device__ __forceinline__ uint32_t key_of_bits(uint32_t bits) { return bits & 0x7FFFFFFFu; }

// Raw bits of element e as fp32 (bf16 widened: its 16 bits on top).
template <int DT> __device__ __forceinline__ uint32_t bits_at(const void *x, int64_t e)
{
    if constexpr (DT == DT_F32)
        return static_cast<const uint32_t *>(x)[e];
    else
        return (uint32_t) static_cast<const uint16_t *>(x)[e] << 16;
}

// One 16-byte vector of raw fp32 bit patterns: 4 fp32 or 8 bf16 values.
template <int DT> struct Vec;
template <> struct Vec<DT_F32> {
    static constexpr int N = 4;
    __device__ static void load(const void *x, int64_t v, uint32_t b[N])
    {
        const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(x) + v);
        b[0] = r.x;
        b[1] = r.y;
        b[2] = r.z;
        b[3] = r.w;
    }
};
template <> struct Vec<DT_BF16> {
    static constexpr int N = 8;
    __device__ static void load(const void *x, int64_t v, uint32_t b[N])
    {
        const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(x) + v);
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            b[2 * j] = w[j] << 16;
            b[2 * j + 1] = w[j] & 0xFFFF0000u;
        }
    }
};

// A whole tile in registers: thread t holds, for round j, the V elements
// starting at tile0 + (j * TT_THREADS + t) * V (so each round's loads are
// coalesced); `valid` masks elements past N.
template <int DT> struct Tile {
    static constexpr int V = Vec<DT>::N;
    static constexpr int ROUNDS = TK_TILE / (TT_THREADS * V);
    uint32_t b[ROUNDS][V];
    __device__ static int64_t first(int64_t tile0, int j) { return tile0 + (int64_t)(j * TT_THREADS + threadIdx.x) * V; }
    __device__ void load(const void *x, int64_t N, bool vec_ok, int64_t tile0)
    {
        if (vec_ok && tile0 + TK_TILE <= N) {
#pragma unroll
            for (int j = 0; j < ROUNDS; ++j)
                Vec<DT>::load(x, first(tile0, j) / V, b[j]);
        } else {
#pragma unroll
            for (int j = 0; j < ROUNDS; ++j)
#pragma unroll
                for (int q = 0; q < V; ++q) {
                    const int64_t e = first(tile0, j) + q;
                    b[j][q] = e < N ? bits_at<DT>(x, e) : 0u;
                }
        }
    }
    __device__ static bool in(int64_t N, int64_t tile0, int j, int q) { return first(tile0, j) + q < N; }
};

// Workgroup-wide exclusive scan of one value per thread (TT_THREADS
// threads); returns the prefix, and the total through `total`.
__device__ __forceinline__ uint32_t wg_exclusive_scan(uint32_t v, uint32_t *s_wave, uint32_t &total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t inc = v;
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_up(inc, d, 64);
        if (lane >= d)
            inc += o;
    }
    if (lane == 63)
        s_wave[wave] = inc;
    __syncthreads();
    uint32_t before = 0, sum = 0;
#pragma unroll
    for (int w = 0; w < TT_WAVES; ++w) {
        const uint32_t s = s_wave[w];
        before += w < wave ? s : 0u;
        sum += s;
    }
    __syncthreads();
    total = sum;
    return before + inc - v;
}

__global__ void topk_init_kernel(TopkWs w, int64_t k)
{
    for (int b = threadIdx.x; b < TK_MAX_BINS; b += blockDim.x)
        w.hist[b] = 0ull;
    for (int r = threadIdx.x; r < TK_REGIONS; r += blockDim.x)
        w.rcount[r] = 0ull;
    if (threadIdx.x == 0) {
        w.st->prefix = 0u;
        w.st->overflow = 0u;
        w.st->rank = k;
    }
}

// LDS histogram of digit (key >> shift) & (bins-1) over keys whose bits
// above the digit equal the prefix; added to the global histogram once per
// workgroup.  Source: the whole input (from_input), or the candidates
// unless they overflowed (then the whole input after all).
template <int DT>
__global__ __launch_bounds__(TK_THREADS) void topk_hist_kernel(const void *x, int64_t N,
                                                               bool vec_ok, TopkWs w, int shift,
                                                               int bits, bool from_input)
{
    __shared__ uint32_t s_hist[TK_WAVES][TK_MAX_BINS];
    const int bins = 1 << bits;
    const uint32_t above =
        (shift + bits >= 31) ? 0u : (0x7FFFFFFFu >> (shift + bits)) << (shift + bits);
    const uint32_t prefix = w.st->prefix & above;
    const bool input = from_input || w.st->overflow;
    const int wave = threadIdx.x >> 6;
    for (int b = threadIdx.x; b < TK_WAVES * bins; b += blockDim.x)
        s_hist[b / bins][b % bins] = 0u;
    __syncthreads();

    uint32_t *h = s_hist[wave];
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    auto count = [&](uint32_t key) {
        if ((key & above) == prefix)
            atomicAdd(&h[(key >> shift) & (uint32_t)(bins - 1)], 1u);
    };
    if (input) {
        constexpr int V = Vec<DT>::N;
        const int64_t nvec = vec_ok ? N / V : 0;
        for (int64_t v = t0; v < nvec; v += stride) {
            uint32_t b[V];
            Vec<DT>::load(x, v, b);
#pragma unroll
            for (int q = 0; q < V; ++q)
                count(key_of_bits(b[q]));
        }
        for (int64_t e = nvec * V + t0; e < N; e += stride)
            count(key_of_bits(bits_at<DT>(x, e)));
    } else {
        // every region's used part; unused slots are skipped
        const int64_t total = (int64_t)TK_REGIONS * w.rcap;
        for (int64_t c = t0; c < total; c += stride) {
            const int64_t r = c / w.rcap;
            if (c - r * w.rcap < (int64_t)w.rcount[r])
                count(w.cand[c].x);
        }
    }
    __syncthreads();
    for (int b = threadIdx.x; b < bins; b += blockDim.x) {
        uint32_t c = 0;
#pragma unroll
        for (int v = 0; v < TK_WAVES; ++v)
            c += s_hist[v][b];
        if (c)
            atomicAdd(&w.hist[b], (unsigned long long)c);
    }
}

// One workgroup: the largest digit d with sum_{u >= d} hist[u] >= rank joins
// the prefix, rank drops by the count of larger digits, and the histogram is
// cleared for the next pass.
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
    // suffix sums from the top bin down: a Hillis-Steele scan, each step
    // reading before any thread writes
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

// Per tile, once the top digit b1 is known: count the keys above bin b1 and
// compact the keys inside it into the candidate buffer (in tile order).
template <int DT>
__global__ __launch_bounds__(TT_THREADS) void topk_split_kernel(const void *x, int64_t N,
                                                                bool vec_ok, TopkWs w)
{
    __shared__ uint32_t s_wave[TT_WAVES];
    __shared__ unsigned long long s_off;
    using TL = Tile<DT>;
    const uint32_t b1 = w.st->prefix >> TK_TOP_SHIFT;
    const int64_t tile0 = (int64_t)blockIdx.x * TK_TILE;
    TL tl;
    tl.load(x, N, vec_ok, tile0);
    uint32_t ndef = 0, ncand = 0;
#pragma unroll
    for (int j = 0; j < TL::ROUNDS; ++j)
#pragma unroll
        for (int q = 0; q < TL::V; ++q) {
            const uint32_t bin = key_of_bits(tl.b[j][q]) >> TK_TOP_SHIFT;
            const bool in = TL::in(N, tile0, j, q);
            ndef += in && bin > b1;
            ncand += in && bin == b1;
        }
    uint32_t tot_def, tot_cand;
    // packed: both counts stay below 2^16 within a tile
    const uint32_t ex = wg_exclusive_scan((ndef << 16) | ncand, s_wave, tot_def);
    tot_cand = tot_def & 0xFFFFu;
    tot_def >>= 16;
    // reserve room in this tile's region (spreading the reservations over
    // TK_REGIONS counters keeps them from queueing on one address)
    const int region = (int)(blockIdx.x % TK_REGIONS);
    if (threadIdx.x == 0) {
        const unsigned long long o = tot_cand ? atomicAdd(&w.rcount[region], (unsigned long long)tot_cand) : 0ull;
        const bool fits = (int64_t)(o + tot_cand) <= w.rcap;
        if (!fits)
            w.st->overflow = 1u;
        s_off = fits ? (unsigned long long)region * w.rcap + o : ~0ull;
        w.def[blockIdx.x] = tot_def;
        w.ccnt[blockIdx.x] = tot_cand;
        w.coff[blockIdx.x] = (unsigned long long)region * w.rcap + o;
    }
    __syncthreads();
    const unsigned long long o = s_off;
    if (o == ~0ull || ncand == 0)
        return;
    unsigned long long pos = o + (ex & 0xFFFFu);
#pragma unroll
    for (int j = 0; j < TL::ROUNDS; ++j)
#pragma unroll
        for (int q = 0; q < TL::V; ++q) {
            const uint32_t key = key_of_bits(tl.b[j][q]);
            if (TL::in(N, tile0, j, q) && (key >> TK_TOP_SHIFT) == b1) {
                w.cand[pos] = u32x2{key, (uint32_t)(TL::first(0, j) + q)};
                ++pos;
            }
        }
}

// Per tile: keys above and equal to the threshold T -- from the tile's
// candidates plus its keys above bin b1, or from the whole tile after an
// overflow.
template <int DT>
__global__ __launch_bounds__(TT_THREADS) void topk_tile_count_kernel(const void *x, int64_t N,
                                                                     bool vec_ok, TopkWs w)
{
    __shared__ uint32_t s_sum[TT_WAVES];
    const uint32_t T = w.st->prefix;
    const int64_t tile0 = (int64_t)blockIdx.x * TK_TILE;
    uint32_t ngt = 0, neq = 0;
    if (w.st->overflow) {
        using TL = Tile<DT>;
        TL tl;
        tl.load(x, N, vec_ok, tile0);
#pragma unroll
        for (int j = 0; j < TL::ROUNDS; ++j)
#pragma unroll
            for (int q = 0; q < TL::V; ++q) {
                const uint32_t key = key_of_bits(tl.b[j][q]);
                const bool in = TL::in(N, tile0, j, q);
                ngt += in && key > T;
                neq += in && key == T;
            }
    } else {
        const unsigned long long c0 = w.coff[blockIdx.x];
        const uint32_t n = w.ccnt[blockIdx.x];
        for (uint32_t c = threadIdx.x; c < n; c += TT_THREADS) {
            const uint32_t key = w.cand[c0 + c].x;
            ngt += key > T;
            neq += key == T;
        }
    }
    uint32_t c = (ngt << 16) | neq;
    for (int d = 32; d > 0; d >>= 1)
        c += __shfl_down(c, d, 64);
    if ((threadIdx.x & 63) == 0)
        s_sum[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t s = 0;
#pragma unroll
        for (int v = 0; v < TT_WAVES; ++v)
            s += s_sum[v];
        w.gt[blockIdx.x] = (s >> 16) + (w.st->overflow ? 0u : w.def[blockIdx.x]);
        w.eq[blockIdx.x] = s & 0xFFFFu;
    }
}

// Workgroup-wide exclusive scan of 64-bit values (TK_SELECT_THREADS threads).
__device__ int64_t big_exclusive_scan(int64_t v, int64_t *s_tmp, int64_t &total)
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
        for (int v = 0; v < TK_SELECT_THREADS / 64; ++v) {
            const int64_t s = s_tmp[v];
            s_tmp[v] = run;
            run += s;
        }
        s_tmp[TK_SELECT_THREADS / 64] = run;
    }
    __syncthreads();
    const int64_t ex = s_tmp[wave] + inc - v;
    total = s_tmp[TK_SELECT_THREADS / 64];
    __syncthreads();
    return ex;
}

// One workgroup, tiles in chunks of 4 per thread (coalesced 16-byte loads):
// tile b keeps take[b] = clamp(r - ties before b, 0, eq[b]) of its ties and
// writes from off[b] = sum over earlier tiles of gt + take.
__global__ __launch_bounds__(TK_SELECT_THREADS) void topk_scan_kernel(int64_t nt, TopkWs w)
{
    __shared__ int64_t s_tmp[TK_SELECT_THREADS / 64 + 1];
    const int64_t r = w.st->rank;
    int64_t ties_carry = 0, sel_carry = 0;
    for (int64_t c0 = 0; c0 < nt; c0 += 4 * TK_SELECT_THREADS) {
        const int64_t b0 = c0 + 4 * (int64_t)threadIdx.x;
        uint32_t g[4] = {0, 0, 0, 0}, e[4] = {0, 0, 0, 0};
        if (b0 < nt) { // arrays are padded to a multiple of 4 tiles
            const u32x4 gv = *reinterpret_cast<const u32x4 *>(w.gt + b0);
            const u32x4 ev = *reinterpret_cast<const u32x4 *>(w.eq + b0);
            const int live = (int)min((int64_t)4, nt - b0);
            g[0] = gv.x; g[1] = live > 1 ? gv.y : 0u; g[2] = live > 2 ? gv.z : 0u; g[3] = live > 3 ? gv.w : 0u;
            e[0] = ev.x; e[1] = live > 1 ? ev.y : 0u; e[2] = live > 2 ? ev.z : 0u; e[3] = live > 3 ? ev.w : 0u;
        }
        int64_t total;
        int64_t tb = ties_carry + big_exclusive_scan((int64_t)e[0] + e[1] + e[2] + e[3], s_tmp, total);
        ties_carry += total;
        uint32_t tk[4];
        int64_t sel = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            tk[i] = (uint32_t)max((int64_t)0, min(r - tb, (int64_t)e[i]));
            tb += e[i];
            sel += g[i] + tk[i];
        }
        int64_t ob = sel_carry + big_exclusive_scan(sel, s_tmp, total);
        sel_carry += total;
        if (b0 < nt) {
            const int live = (int)min((int64_t)4, nt - b0);
            for (int i = 0; i < live; ++i) {
                w.take[b0 + i] = tk[i];
                w.off[b0 + i] = ob;
                ob += g[i] + tk[i];
            }
        }
    }
}

// Per tile: the kept entries in index order.  The tile is loaded whole into
// registers; every round's elements get their rank among the tile's kept
// entries from wave scans of the packed (above, tie) counts and one exchange
// of the per-wave round totals in LDS.  The first TK_STAGE kept entries are
// staged in LDS and then written out as two contiguous runs; any beyond that
// (a tile keeping more than a quarter of its elements) go straight out.
constexpr int TK_STAGE = 2048;

template <int DT>
__global__ __launch_bounds__(TT_THREADS) void topk_write_kernel(const void *x, int64_t N,
                                                                bool vec_ok, TopkWs w, int64_t k_out,
                                                                int64_t *idx_out, float *val_out)
{
    using TL = Tile<DT>;
    __shared__ uint32_t s_tot[TL::ROUNDS][TT_WAVES];
    __shared__ uint32_t s_idx[TK_STAGE];
    __shared__ float s_val[TK_STAGE];
    const uint32_t T = w.st->prefix;
    const int64_t tile0 = (int64_t)blockIdx.x * TK_TILE;
    const uint32_t tk = w.take[blockIdx.x];
    const int64_t base = w.off[blockIdx.x];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    TL tl;
    tl.load(x, N, vec_ok, tile0);
    uint32_t inc[TL::ROUNDS];
#pragma unroll
    for (int j = 0; j < TL::ROUNDS; ++j) {
        uint32_t ngt = 0, neq = 0;
#pragma unroll
        for (int q = 0; q < TL::V; ++q) {
            const uint32_t key = key_of_bits(tl.b[j][q]);
            const bool in = TL::in(N, tile0, j, q);
            ngt += in && key > T;
            neq += in && key == T;
        }
        uint32_t v = (ngt << 16) | neq;
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t o = __shfl_up(v, d, 64);
            if (lane >= d)
                v += o;
        }
        inc[j] = v;
        if (lane == 63)
            s_tot[j][wave] = v;
    }
    __syncthreads();
    uint32_t carry = 0; // packed counts of the rounds before j
    uint32_t kept_total = 0;
#pragma unroll
    for (int j = 0; j < TL::ROUNDS; ++j) {
        uint32_t before = 0, round_total = 0;
#pragma unroll
        for (int v = 0; v < TT_WAVES; ++v) {
            const uint32_t t = s_tot[j][v];
            before += v < wave ? t : 0u;
            round_total += t;
        }
        // this thread's exclusive prefix: everything before it in this round;
        // the lanes below it come from the inclusive scan of the lane below
        // (the shuffle runs on every lane: a disabled source lane would give
        // no data)
        const uint32_t below = __shfl_up(inc[j], 1, 64);
        uint32_t run = carry + before + (lane > 0 ? below : 0u);
        carry += round_total;
        uint32_t gt_before = run >> 16, eq_before = run & 0xFFFFu;
#pragma unroll
        for (int q = 0; q < TL::V; ++q) {
            const uint32_t bits = tl.b[j][q];
            const uint32_t key = key_of_bits(bits);
            if (!TL::in(N, tile0, j, q) || key < T)
                continue;
            const bool above = key > T;
            const bool kept = above || eq_before < tk;
            // rank among the tile's kept entries
            const uint32_t r = gt_before + min(eq_before, tk);
            if (above)
                ++gt_before;
            else
                ++eq_before;
            if (!kept)
                continue;
            const uint32_t local = (uint32_t)(TL::first(0, j) + q);
            if (r < TK_STAGE) {
                s_idx[r] = local;
                s_val[r] = __uint_as_float(bits);
            } else if (base + r < k_out) {
                // the bound keeps inconsistent counts from writing out of range
                idx_out[base + r] = tile0 + local;
                val_out[base + r] = __uint_as_float(bits);
            }
        }
    }
    kept_total = (carry >> 16) + min(carry & 0xFFFFu, tk);
    __syncthreads();
    const int n = (int)min((uint32_t)TK_STAGE, kept_total);
    for (int i = threadIdx.x; i < n; i += TT_THREADS) {
        if (base + i < k_out) {
            idx_out[base + i] = tile0 + s_idx[i];
            val_out[base + i] = s_val[i];
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
    const TopkWs w = carve(ws, N);
    const int64_t nt = (N + TK_TILE - 1) / TK_TILE;
    const bool vec_ok = (reinterpret_cast<uintptr_t>(x) & 15u) == 0;
    const unsigned full_grid = grid_of(N / Vec<DT>::N + 1, (int64_t)cus * 4);
    const unsigned cand_grid = grid_of((int64_t)TK_REGIONS * w.rcap, (int64_t)cus * 4);

    topk_init_kernel<<<1, 256, 0, s>>>(w, k);
    // digit 1: key bits 30..20, over the whole input
    topk_hist_kernel<DT><<<full_grid, TK_THREADS, 0, s>>>(x, N, vec_ok, w, TK_TOP_SHIFT, 11, true);
    topk_select_kernel<<<1, TK_SELECT_THREADS, 0, s>>>(w.hist, w.st, TK_TOP_SHIFT, 11);
    topk_split_kernel<DT><<<(unsigned)nt, TT_THREADS, 0, s>>>(x, N, vec_ok, w);
    // digits 2 (bits 19..9) and, for fp32, 3 (bits 8..0), over the candidates
    // (a bf16 key has zeros below bit 16, so two digits decide it); after an
    // overflow the grid covers the whole input
    const unsigned later_grid = full_grid > cand_grid ? full_grid : cand_grid;
    topk_hist_kernel<DT><<<later_grid, TK_THREADS, 0, s>>>(x, N, vec_ok, w, 9, 11, false);
    topk_select_kernel<<<1, TK_SELECT_THREADS, 0, s>>>(w.hist, w.st, 9, 11);
    if (DT == DT_F32) {
        topk_hist_kernel<DT><<<later_grid, TK_THREADS, 0, s>>>(x, N, vec_ok, w, 0, 9, false);
        topk_select_kernel<<<1, TK_SELECT_THREADS, 0, s>>>(w.hist, w.st, 0, 9);
    }
    topk_tile_count_kernel<DT><<<(unsigned)nt, TT_THREADS, 0, s>>>(x, N, vec_ok, w);
    topk_scan_kernel<<<1, TK_SELECT_THREADS, 0, s>>>(nt, w);
    topk_write_kernel<DT><<<(unsigned)nt, TT_THREADS, 0, s>>>(x, N, vec_ok, w, k, idx_out, val_out);
    return hipGetLastError();
}

} // namespace

size_t topk_workspace_bytes(int64_t N)
{
    const int64_t ntp = round4((N + TK_TILE - 1) / TK_TILE);
    return (size_t)TK_MAX_BINS * 8 + 256 + (size_t)TK_REGIONS * 8 + (size_t)ntp * (8 + 8 + 4 * 5) +
           (size_t)TK_REGIONS * region_capacity(N) * 8;
}

hipError_t launch_topk(const void *x, int dt, int64_t N, int64_t k, int64_t *idx_out,
                       float *val_out, void *ws, int cus, hipStream_t s)
{
    return dt == DT_F32 ? topk_run<DT_F32>(x, N, k, idx_out, val_out, ws, cus, s)
                        : topk_run<DT_BF16>(x, N, k, idx_out, val_out, ws, cus, s);
}

} // namespace fa
