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
// The k-th largest key T is found exactly by radix select, most significant
// digit first, in digits of 11, 11 and 9 bits (bf16 keys have 15 bits: two
// digits decide them); each tile of TK_TILE elements then writes its kept
// entries from an output offset given by a scan of the per-tile counts.
//
// Sampled path (the usual one).  A systematic sample of about 2^20 keys
// bounds T from both sides: K_lo and K_hi are the sample's order statistics
// a wide margin (8 binomial standard deviations plus 32) below and above
// T's expected rank, rounded outwards to 22-bit key prefixes.  One pass over
// the update then, per tile, counts the keys above K_hi, compacts the keys
// inside [K_lo, K_hi] -- the candidates, well under one per cent of the input
// for smooth data -- and, when k is small enough for it to pay, copies every
// key at or above K_lo with its position into the tile's segment of a
// staging buffer, in index order.  One workgroup checks that the range holds
// T (fewer than k keys above K_hi, at least k at or above K_lo, no buffer
// overflowed); the digits of T are chosen from histograms of the candidates
// only, and the ordered write reads the staging segments (or, without them,
// the update).  The update is read once (twice without staging).
//
// Full path.  When the check fails, the sample cannot bound T (k near N) or
// the caller asks for it, a flag in the workspace sends every later kernel
// down three passes over the update: a histogram of the top digit; a split
// that counts the keys above T's top-digit bin and compacts those inside it
// as candidates (or, when they outgrow their buffer, a second flag that makes
// the later kernels use the whole input again); and the ordered write.  The
// result is the same on both paths.  No workgroup ever waits on another.
#include <hip/hip_runtime.h>
#include <math.h>

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
constexpr int TK_SUB_SHIFT = 9;  // second digit: key bits 19..9
constexpr int TK_REGIONS = 256;  // candidate / staging regions, each with its own counter
constexpr int TK_CSTRIDE = 16;   // region counters lie 128 bytes apart: atomics on
                                 // different regions never share a cache line
constexpr int TK_STAGE = 2048;   // entries a per-tile kernel stages in LDS
constexpr int TK_SCAN_CHUNK = 4 * 256; // tiles per workgroup of the offset scan
constexpr int64_t TK_SAMPLE_KEYS = 1 << 20;

using u32x2 = __attribute__((ext_vector_type(2))) unsigned int;
using u32x4 = __attribute__((ext_vector_type(4))) unsigned int;

struct TopkState {
    uint32_t prefix;   // key bits chosen so far (the threshold T at the end)
    uint32_t overflow; // full path: candidates did not fit, use the whole input
    int64_t rank;      // keys matching `prefix` still to be kept
    uint32_t fast;     // the sampled range held T: the sampled path is on
    uint32_t ranged;   // the sample gave a range [klo, khi]
    uint32_t fov;      // sampled path: a candidate or staging region overflowed
    uint32_t klo, khi;
    uint32_t sbin_hi, sbin_lo;  // sample: top-digit bins of the two order statistics
    int64_t srank_hi, srank_lo; // and their ranks inside those bins
    // sampled path with rel set: T's digits are those of d = (key - klo) >> g,
    // the upper one d >> sh1 (found first, kept in dprefix) and the lower sh1
    // bits; with rel clear (a range too wide) the candidates' absolute digits
    uint32_t rel, g, sh1, dprefix;
};
static_assert(sizeof(TopkState) <= 256, "state slot");

// Where the pieces of the workspace live.
struct TopkWs {
    unsigned long long *hist; // 2 x TK_MAX_BINS
    TopkState *st;
    unsigned long long *rcnt;   // per region, TK_CSTRIDE apart: (staging entries << 32) |
                                // candidates reserved (the full path: candidates only)
    int64_t *off;               // per tile: first output position
    unsigned long long *coff;   // per tile: first candidate
    unsigned long long *toff;   // per tile: first staging entry
    uint32_t *gt, *eq;          // per tile: keys above / equal to T
    uint32_t *take;             // per tile: ties kept
    uint32_t *def;              // per tile: keys above the candidates
    uint32_t *ccnt;             // per tile: candidates
    uint32_t *tcnt;             // per tile: staging entries
    int64_t *ch_eq, *ch_gt;     // per scan chunk: sums of eq and gt
    int64_t *ch_ties, *ch_off;  // per scan chunk: ties before it, first output position
    u32x2 *cand;                // (key, position in tile), TK_REGIONS regions of rcap
    int64_t rcap;
    void *sval;                 // staged value bits (uint32 for fp32, uint16 for bf16) and
    uint16_t *sloc;             // position in tile, parallel arrays: TK_REGIONS regions of tcap
    int64_t tcap;
};

__host__ __device__ constexpr int64_t round4(int64_t n) { return (n + 3) / 4 * 4; }

// A staged entry is the value's bits (4 bytes for fp32, 2 for bf16) and its
// 2-byte position in the tile.  Staging pays when writing and re-reading the
// entries costs less than a second read of the update: 12 k < 4 N for fp32,
// 8 k < 2 N for bf16.
constexpr int64_t staged_bytes(int dt) { return dt == DT_F32 ? 6 : 4; }
bool staging_pays(int64_t N, int64_t k, int dt) { return dt == DT_F32 ? 3 * k < N : 4 * k < N; }

struct Sizes {
    int64_t nt, ntp, nch, rcap, tcap;
    size_t bytes;
};

Sizes sizes_of(int64_t N, int64_t k, int dt)
{
    Sizes s;
    s.nt = (N + TK_TILE - 1) / TK_TILE;
    s.ntp = round4(s.nt);
    s.nch = (s.nt + TK_SCAN_CHUNK - 1) / TK_SCAN_CHUNK;
    // candidates: N/16 + 64Ki in all; staging: k + N/64 + 64Ki in all
    s.rcap = (N / 16 + 65536 + TK_REGIONS - 1) / TK_REGIONS;
    s.tcap = staging_pays(N, k, dt) ? (k + N / 64 + 65536 + TK_REGIONS - 1) / TK_REGIONS : 0;
    s.bytes = (size_t)2 * TK_MAX_BINS * 8 + 256 + (size_t)TK_REGIONS * TK_CSTRIDE * 8 +
              (size_t)s.ntp * (3 * 8 + 6 * 4) + (size_t)s.nch * 4 * 8 +
              (size_t)TK_REGIONS * s.rcap * 8 + (size_t)TK_REGIONS * s.tcap * staged_bytes(dt);
    return s;
}

TopkWs carve(void *ws, const Sizes &s, int dt)
{
    char *w = static_cast<char *>(ws);
    TopkWs p;
    p.hist = reinterpret_cast<unsigned long long *>(w);
    w += 2 * TK_MAX_BINS * 8;
    p.st = reinterpret_cast<TopkState *>(w);
    w += 256;
    p.rcnt = reinterpret_cast<unsigned long long *>(w);
    w += TK_REGIONS * TK_CSTRIDE * 8;
    p.off = reinterpret_cast<int64_t *>(w);
    p.coff = reinterpret_cast<unsigned long long *>(p.off + s.ntp);
    p.toff = p.coff + s.ntp;
    w += s.ntp * 3 * 8;
    p.gt = reinterpret_cast<uint32_t *>(w); // 16-byte aligned: the scan loads 4 at a time
    p.eq = p.gt + s.ntp;
    p.take = p.eq + s.ntp;
    p.def = p.take + s.ntp;
    p.ccnt = p.def + s.ntp;
    p.tcnt = p.ccnt + s.ntp;
    w += s.ntp * 6 * 4;
    p.ch_eq = reinterpret_cast<int64_t *>(w);
    p.ch_gt = p.ch_eq + s.nch;
    p.ch_ties = p.ch_gt + s.nch;
    p.ch_off = p.ch_ties + s.nch;
    w += s.nch * 4 * 8;
    p.cand = reinterpret_cast<u32x2 *>(w);
    p.rcap = s.rcap;
    p.sval = p.cand + TK_REGIONS * s.rcap;
    p.sloc = reinterpret_cast<uint16_t *>(static_cast<char *>(p.sval) +
                                          TK_REGIONS * s.tcap * (staged_bytes(dt) - 2));
    p.tcap = s.tcap;
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
// coalesced).  Elements past N read as 0 (key 0); in index order they come
// after every element of the tile that exists, so a kernel needs no
// per-element bounds test: it takes the pad() of them out of any count whose
// predicate key 0 meets, and bounds its writes by the corrected count.  The
// thread index is passed through an empty asm statement so that a loop over
// tiles recomputes per-element offsets (one add each) rather than keeping
// them all in registers.
template <int DT> struct Tile {
    static constexpr int V = Vec<DT>::N;
    static constexpr int ROUNDS = TK_TILE / (TT_THREADS * V);
    uint32_t b[ROUNDS][V];
    uint32_t t;   // this thread's index
    uint32_t lim; // elements of the tile below N
    __device__ uint32_t local(int j, int q) const { return (uint32_t)(j * TT_THREADS + t) * V + q; }
    __device__ uint32_t pad() const { return (uint32_t)TK_TILE - lim; }
    // Before a second pass over the tile: the values pass through empty asm
    // statements, so the pass derives keys and compares from the raw bits
    // again rather than keeping the first pass's results live.
    __device__ void reuse()
    {
#pragma unroll
        for (int j = 0; j < ROUNDS; ++j)
#pragma unroll
            for (int q = 0; q < V; ++q)
                asm volatile("" : "+v"(b[j][q]));
        asm volatile("" : "+v"(t));
    }
    __device__ void load(const void *x, int64_t N, bool vec_ok, int64_t tile0)
    {
        t = threadIdx.x;
        asm volatile("" : "+v"(t));
        const int64_t left = N - tile0;
        lim = left < TK_TILE ? (uint32_t)left : (uint32_t)TK_TILE;
        if (vec_ok && lim == (uint32_t)TK_TILE) {
#pragma unroll
            for (int j = 0; j < ROUNDS; ++j)
                Vec<DT>::load(x, tile0 / V + (j * TT_THREADS + t), b[j]);
        } else {
#pragma unroll
            for (int j = 0; j < ROUNDS; ++j)
#pragma unroll
                for (int q = 0; q < V; ++q) {
                    const uint32_t l = local(j, q);
                    b[j][q] = l < lim ? bits_at<DT>(x, tile0 + l) : 0u;
                }
        }
    }
};

// Inclusive scan over the 64 lanes of a wave with DPP adds: Hillis-Steele
// inside each row of 16 lanes (row_shr 1, 2, 4, 8; lanes with no source read
// 0), then lane 15 of rows 0 and 2 is added into rows 1 and 3 (row_bcast:15)
// and lane 31 into rows 2 and 3 (row_bcast:31).  Lanes a row mask leaves out
// read the `old` operand, 0.  Every lane of the wave must be active.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v)
{
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true); // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true); // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true); // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true); // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false); // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false); // row_bcast:31
    return v;
}

// Workgroup-wide exclusive scan of one 64-bit value per thread (THREADS
// threads); returns the prefix, and the total through `total`.  Ends with a
// barrier, so s_tmp may be reused at once.
template <int THREADS>
__device__ int64_t block_exclusive_scan64(int64_t v, int64_t *s_tmp, int64_t &total)
{
    constexpr int WAVES = THREADS / 64;
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
        for (int u = 0; u < WAVES; ++u) {
            const int64_t s = s_tmp[u];
            s_tmp[u] = run;
            run += s;
        }
        s_tmp[WAVES] = run;
    }
    __syncthreads();
    const int64_t ex = s_tmp[wave] + inc - v;
    total = s_tmp[WAVES];
    __syncthreads();
    return ex;
}

__global__ void topk_init_kernel(TopkWs w, int64_t k)
{
    for (int b = threadIdx.x; b < 2 * TK_MAX_BINS; b += blockDim.x)
        w.hist[b] = 0ull;
    for (int r = threadIdx.x; r < TK_REGIONS; r += blockDim.x) {
        w.rcnt[r * TK_CSTRIDE] = 0ull;
    }
    if (threadIdx.x == 0) {
        TopkState s = {};
        s.rank = k;
        *w.st = s;
    }
}

// ------------------------------------------------------------ the sample

// Histograms of the sampled keys.  Sample unit s (0 <= s < mu) is unit
// floor(s * units / mu) of the update: one 16-byte vector (vec_units) or one
// element.  Level 1: the top digit (bits 30..20) into hist[0..2048).  Level
// 2: the second digit (bits 19..9) of the keys whose top digit is the bin of
// the upper order statistic (into hist[0..2048)) and of the lower one (into
// hist[2048..4096)).
template <int DT>
__global__ __launch_bounds__(TK_THREADS) void topk_sample_hist_kernel(const void *x, bool vec_units,
                                                                      int64_t units, int64_t mu,
                                                                      TopkWs w, int level, bool has_hi)
{
    __shared__ uint32_t s_h[2][TK_MAX_BINS];
    for (int b = threadIdx.x; b < 2 * TK_MAX_BINS; b += blockDim.x)
        s_h[b / TK_MAX_BINS][b % TK_MAX_BINS] = 0u;
    __syncthreads();
    const uint32_t bhi = level == 2 ? w.st->sbin_hi : 0u;
    const uint32_t blo = level == 2 ? w.st->sbin_lo : 0u;
    auto count = [&](uint32_t key) {
        const uint32_t top = key >> TK_TOP_SHIFT;
        if (level == 1) {
            atomicAdd(&s_h[0][top], 1u);
        } else {
            const uint32_t d = (key >> TK_SUB_SHIFT) & (TK_MAX_BINS - 1);
            if (has_hi && top == bhi)
                atomicAdd(&s_h[0][d], 1u);
            if (top == blo)
                atomicAdd(&s_h[1][d], 1u);
        }
    };
    // floor(s * units / mu) without overflow: s * q + floor(s * rem / mu);
    // SU units' loads are issued before any is counted
    constexpr int SU = 4;
    const int64_t q = units / mu, rem = units % mu;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    auto unit = [&](int64_t s) { return s * q + (s * rem) / mu; };
    int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (vec_units) {
        constexpr int V = Vec<DT>::N;
        for (; s + (SU - 1) * stride < mu; s += SU * stride) {
            uint32_t b[SU][V];
#pragma unroll
            for (int j = 0; j < SU; ++j)
                Vec<DT>::load(x, unit(s + j * stride), b[j]);
#pragma unroll
            for (int j = 0; j < SU; ++j)
#pragma unroll
                for (int i = 0; i < V; ++i)
                    count(key_of_bits(b[j][i]));
        }
        for (; s < mu; s += stride) {
            uint32_t b[V];
            Vec<DT>::load(x, unit(s), b);
#pragma unroll
            for (int i = 0; i < V; ++i)
                count(key_of_bits(b[i]));
        }
    } else {
        for (; s < mu; s += stride)
            count(key_of_bits(bits_at<DT>(x, unit(s))));
    }
    __syncthreads();
    for (int b = threadIdx.x; b < TK_MAX_BINS; b += blockDim.x) {
        const uint32_t c0 = s_h[0][b];
        if (c0)
            atomicAdd(&w.hist[b], (unsigned long long)c0);
        if (level == 2) {
            const uint32_t c1 = s_h[1][b];
            if (c1)
                atomicAdd(&w.hist[TK_MAX_BINS + b], (unsigned long long)c1);
        }
    }
}

// The bin b of hist[0..bins) holding the rank-th largest key, counting from
// the top bin down: suffix(b) >= rank > suffix(b + 1), with suffix(b) the sum
// of hist[u] for u >= b (there is one when 1 <= rank <= suffix(0)); *rem
// gets rank - suffix(b + 1), the rank left inside the bin.  Every thread
// gets both; -1 when there is no such bin.  Thread t holds bins
// bins-1-2t and bins-2-2t, so a prefix scan over threads is the suffix scan
// over bins.  TK_SELECT_THREADS threads; ends with a barrier.
__device__ int select_bin(const unsigned long long *hist, int bins, int64_t rank, int64_t *rem,
                          unsigned long long *s_wtot, int *s_bin, int64_t *s_rem)
{
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int hi = bins - 1 - 2 * t, lo = hi - 1;
    const unsigned long long hh = hi >= 0 ? hist[hi] : 0ull, hl = lo >= 0 ? hist[lo] : 0ull;
    const unsigned long long pair = hh + hl;
    unsigned long long inc = pair;
    for (int d = 1; d < 64; d <<= 1) {
        const unsigned long long o = __shfl_up(inc, d, 64);
        if (lane >= d)
            inc += o;
    }
    if (lane == 63)
        s_wtot[wave] = inc;
    if (t == 0)
        *s_bin = -1;
    __syncthreads();
    for (int v = 0; v < wave; ++v)
        inc += s_wtot[v];
    // suffix(hi + 1) = ex, suffix(hi) = ex + hh = suffix(lo + 1), suffix(lo) = inc
    const int64_t ex = (int64_t)(inc - pair), mid = ex + (int64_t)hh, all = (int64_t)inc;
    if (hi >= 0 && mid >= rank && ex < rank) {
        *s_bin = hi;
        *s_rem = rank - ex;
    }
    if (lo >= 0 && all >= rank && mid < rank) {
        *s_bin = lo;
        *s_rem = rank - mid;
    }
    __syncthreads();
    const int b = *s_bin;
    *rem = *s_rem;
    __syncthreads();
    return b;
}

// One workgroup.  Level 1: the top-digit bins holding the sample's r_hi-th
// and r_lo-th largest keys (ranks from the top, 1-based) and the ranks left
// inside them.  Level 2: their second digits, giving K_hi = the upper one's
// 22-bit prefix with all lower bits set (no upper bound when !has_hi) and
// K_lo = the lower one's prefix with the lower bits clear.  The histograms
// are cleared for the next pass.
__global__ __launch_bounds__(TK_SELECT_THREADS) void topk_sample_select_kernel(TopkWs w, int level,
                                                                               bool has_hi,
                                                                               int64_t r_hi,
                                                                               int64_t r_lo)
{
    __shared__ unsigned long long s_wtot[TK_SELECT_THREADS / 64];
    __shared__ int s_bin;
    __shared__ int64_t s_rem;
    TopkState *st = w.st;
    const int t = threadIdx.x;
    int64_t rem_hi = 0, rem_lo = 0;
    if (level == 1) {
        const int bh = has_hi ? select_bin(w.hist, TK_MAX_BINS, r_hi, &rem_hi, s_wtot, &s_bin, &s_rem) : 0;
        const int bl = select_bin(w.hist, TK_MAX_BINS, r_lo, &rem_lo, s_wtot, &s_bin, &s_rem);
        if (t == 0) {
            st->sbin_hi = bh < 0 ? 0u : (uint32_t)bh;
            st->srank_hi = has_hi && bh >= 0 ? rem_hi : 0;
            st->sbin_lo = bl < 0 ? 0u : (uint32_t)bl;
            st->srank_lo = bl >= 0 ? rem_lo : 0;
            st->ranged = bh >= 0 && bl >= 0;
        }
        for (int b = t; b < TK_MAX_BINS; b += blockDim.x)
            w.hist[b] = 0ull;
    } else {
        // read before the barriers: thread 0 rewrites `ranged` at the end
        const int64_t sr_hi = st->srank_hi, sr_lo = st->srank_lo;
        const uint32_t bh = st->sbin_hi, bl = st->sbin_lo;
        const bool ok = st->ranged != 0u;
        int dh = TK_MAX_BINS - 1;
        if (has_hi)
            dh = select_bin(w.hist, TK_MAX_BINS, sr_hi, &rem_hi, s_wtot, &s_bin, &s_rem);
        const int dl = select_bin(w.hist + TK_MAX_BINS, TK_MAX_BINS, sr_lo, &rem_lo, s_wtot, &s_bin, &s_rem);
        if (t == 0) {
            st->khi = has_hi ? (bh << TK_TOP_SHIFT) | ((uint32_t)max(dh, 0) << TK_SUB_SHIFT) |
                                   ((1u << TK_SUB_SHIFT) - 1u)
                             : 0x7FFFFFFFu;
            const uint32_t klo = (bl << TK_TOP_SHIFT) | ((uint32_t)max(dl, 0) << TK_SUB_SHIFT);
            st->klo = klo;
            // a range down to key 0 (an update mostly of zeros) takes the
            // full path: the split reads positions past N as key 0 and
            // relies on klo > 0 never to choose them
            st->ranged = ok && dh >= 0 && dl >= 0 && klo > 0u;
        }
        for (int b = t; b < 2 * TK_MAX_BINS; b += blockDim.x)
            w.hist[b] = 0ull;
    }
}

// ------------------------------------------------------------ sampled path

// A staged entry: the value (bf16 keeps its 16 bits) and its position.
template <int DT> __device__ __forceinline__ void stage_put(const TopkWs &w, uint64_t at, uint32_t bits,
                                                            uint32_t local)
{
    if constexpr (DT == DT_F32)
        static_cast<uint32_t *>(w.sval)[at] = bits;
    else
        static_cast<uint16_t *>(w.sval)[at] = (uint16_t)(bits >> 16);
    w.sloc[at] = (uint16_t)local;
}
template <int DT> __device__ __forceinline__ uint32_t stage_bits(const TopkWs &w, uint64_t at)
{
    if constexpr (DT == DT_F32)
        return static_cast<const uint32_t *>(w.sval)[at];
    else
        return (uint32_t) static_cast<const uint16_t *>(w.sval)[at] << 16;
}

// Per tile, with the range [klo, khi] known: count the keys above khi,
// compact the keys inside the range into the tile's candidate segment and,
// with staging, every key at or above klo with its position into the tile's
// staging segment -- both in index order.  Segments are reserved in the
// tile's region (tile mod TK_REGIONS) with one atomic each; a region that
// runs out sets `fov` and the check sends the call down the full path.
//
// Wave w of the workgroup takes the tile's elements [w S, (w + 1) S),
// S = TK_TILE / TT_WAVES, as SPLIT_COLS columns of 64 consecutive elements,
// lane l holding element l of each column.  Index order is then column
// order, lane order inside a column, so an element's rank among the chosen
// ones is a wave-uniform running count plus the number of chosen lanes below
// it in its column's ballot: a few instructions per column of 64 elements,
// where ranking each lane's own consecutive elements one after another took
// a divergent branch per element.
constexpr int SPLIT_COLS = TK_TILE / TT_THREADS;
constexpr int SPLIT_SPAN = TK_TILE / TT_WAVES;

__device__ __forceinline__ uint32_t lanes_below(uint64_t m)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Raw buffer over `bytes` bytes from p: a load past them returns 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t split_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, 0x00020000);
}

constexpr int SPLIT_CAND = 1024; // candidates a tile gathers in LDS (more go out directly)

template <int DT>
__device__ __forceinline__ void split_tile(const void *x, int64_t tile, int64_t tile0, uint32_t lim,
                                           uint32_t lo, uint32_t hi, const TopkWs &w, bool staging,
                                           uint32_t *s_ge, uint32_t *s_in,
                                           unsigned long long *s_seg, uint32_t *s_bits,
                                           uint16_t *s_loc, uint32_t *s_ckey, uint16_t *s_cloc)
{
    constexpr uint32_t EB = DT == DT_F32 ? 4 : 2; // bytes per element
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t first = (uint32_t)wave * SPLIT_SPAN + lane; // local position in column 0
    // elements past N read as 0 through the buffer's range: key 0 is below
    // lo (> 0 on this path), so they are never chosen
    const auto xr = split_rsrc(static_cast<const char *>(x) + tile0 * EB, lim * EB);
    uint32_t b[SPLIT_COLS];
#pragma unroll
    for (int c = 0; c < SPLIT_COLS; ++c) {
        if constexpr (DT == DT_F32)
            b[c] = __builtin_amdgcn_raw_buffer_load_b32(xr, (int)(first * EB), c * 64 * EB, 2);
        else
            b[c] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(xr, (int)(first * EB), c * 64 * EB, 2) << 16;
    }
    uint32_t n_ge = 0, n_in = 0; // this wave's counts (wave-uniform)
#pragma unroll
    for (int c = 0; c < SPLIT_COLS; ++c) {
        const uint32_t key = key_of_bits(b[c]);
        n_ge += (uint32_t)__popcll(__builtin_amdgcn_ballot_w64(key >= lo));
        n_in += (uint32_t)__popcll(__builtin_amdgcn_ballot_w64(key >= lo && key <= hi));
    }
    if (lane == 0) {
        s_ge[wave] = n_ge;
        s_in[wave] = n_in;
    }
    __syncthreads();
    uint32_t t_ge = 0, t_in = 0, rt = 0, rc = 0;
#pragma unroll
    for (int v = 0; v < TT_WAVES; ++v) {
        const uint32_t g = s_ge[v], i = s_in[v];
        t_ge += g;
        t_in += i;
        rt += v < wave ? g : 0u; // ranks of this wave's first chosen elements
        rc += v < wave ? i : 0u;
    }
    // wave-uniform, kept in scalar registers
    t_ge = __builtin_amdgcn_readfirstlane(t_ge);
    t_in = __builtin_amdgcn_readfirstlane(t_in);
    rt = __builtin_amdgcn_readfirstlane(rt);
    rc = __builtin_amdgcn_readfirstlane(rc);
    if (threadIdx.x == 0) {
        // The segments are reserved while the tile ranks its entries into
        // LDS: the atomic's round trip overlaps that pass, and only the
        // copy-out below needs the reserved offsets.  One atomic reserves
        // both segments; the staging count runs with or without staging: the
        // check reads the keys >= klo from it.
        const int region = (int)(tile % TK_REGIONS);
        const unsigned long long o =
            t_ge ? atomicAdd(&w.rcnt[region * TK_CSTRIDE], ((unsigned long long)t_ge << 32) | t_in) : 0ull;
        const unsigned long long ot = o >> 32, oc = o & 0xFFFFFFFFull;
        const bool tfits = !staging || (int64_t)(ot + t_ge) <= w.tcap;
        const bool cfits = (int64_t)(oc + t_in) <= w.rcap;
        if (!tfits || !cfits)
            w.st->fov = 1u;
        s_seg[0] = staging && tfits ? (unsigned long long)region * w.tcap + ot : ~0ull;
        s_seg[1] = cfits ? (unsigned long long)region * w.rcap + oc : ~0ull;
        w.def[tile] = t_ge - t_in;
        w.ccnt[tile] = t_in;
        w.coff[tile] = (unsigned long long)region * w.rcap + oc;
        w.tcnt[tile] = t_ge;
        w.toff[tile] = staging ? (unsigned long long)region * w.tcap + ot : 0ull;
    }
    // the ranking pass derives keys and tests from the raw bits again rather
    // than keeping the count pass's per-column results live across the
    // barrier (64 more registers)
#pragma unroll
    for (int c = 0; c < SPLIT_COLS; ++c)
        asm volatile("" : "+v"(b[c]));
#pragma unroll
    for (int c = 0; c < SPLIT_COLS; ++c) {
        const uint32_t key = key_of_bits(b[c]);
        const bool ge = key >= lo;
        const bool in = ge && key <= hi;
        const uint64_t mg = __builtin_amdgcn_ballot_w64(ge), mi = __builtin_amdgcn_ballot_w64(in);
        // formed here from an opaque copy: kept for all columns (they do
        // not change from tile to tile) they would hold 32 registers
        uint32_t local = first;
        asm volatile("" : "+v"(local));
        local += c * 64;
        if (ge) {
            const uint32_t r = rt + lanes_below(mg);
            if (r < TK_STAGE) {
                s_bits[r] = b[c];
                s_loc[r] = (uint16_t)local;
            }
        }
        if (in) {
            const uint32_t r = rc + lanes_below(mi);
            if (r < SPLIT_CAND) {
                s_ckey[r] = key;
                s_cloc[r] = (uint16_t)local;
            }
        }
        rt += (uint32_t)__popcll(mg);
        rc += (uint32_t)__popcll(mi);
    }
    __syncthreads();
    const unsigned long long toff = s_seg[0], coff = s_seg[1];
    if (toff != ~0ull) {
        const uint32_t n = min((uint32_t)TK_STAGE, t_ge);
        for (uint32_t i = threadIdx.x; i < n; i += TT_THREADS)
            stage_put<DT>(w, toff + i, s_bits[i], s_loc[i]);
    }
    if (coff != ~0ull) {
        const uint32_t n = min((uint32_t)SPLIT_CAND, t_in);
        for (uint32_t i = threadIdx.x; i < n; i += TT_THREADS)
            w.cand[coff + i] = u32x2{s_ckey[i], (uint32_t)s_cloc[i]};
    }
    // A tile with more entries than LDS holds (over a quarter of it staged,
    // or an eighth of it candidates) writes the rest straight out.
    if ((t_ge > TK_STAGE && toff != ~0ull) || (t_in > SPLIT_CAND && coff != ~0ull)) {
        uint32_t qt = __builtin_amdgcn_readfirstlane(rt - n_ge), qc = __builtin_amdgcn_readfirstlane(rc - n_in);
#pragma unroll
        for (int c = 0; c < SPLIT_COLS; ++c)
            asm volatile("" : "+v"(b[c]));
#pragma unroll
        for (int c = 0; c < SPLIT_COLS; ++c) {
            const uint32_t key = key_of_bits(b[c]);
            const bool ge = key >= lo;
            const bool in = ge && key <= hi;
            const uint64_t mg = __builtin_amdgcn_ballot_w64(ge), mi = __builtin_amdgcn_ballot_w64(in);
            uint32_t local = first;
            asm volatile("" : "+v"(local));
            local += c * 64;
            if (ge && toff != ~0ull) {
                const uint32_t r = qt + lanes_below(mg);
                if (r >= TK_STAGE)
                    stage_put<DT>(w, toff + r, b[c], local);
            }
            if (in && coff != ~0ull) {
                const uint32_t r = qc + lanes_below(mi);
                if (r >= SPLIT_CAND)
                    w.cand[coff + r] = u32x2{key, local};
            }
            qt += (uint32_t)__popcll(mg);
            qc += (uint32_t)__popcll(mi);
        }
    }
    __syncthreads(); // the LDS arrays are reused by the next tile
}

template <int DT>
__global__ __launch_bounds__(TT_THREADS) void topk_split_range_kernel(const void *x, int64_t N, int64_t nt,
                                                                      TopkWs w, bool staging)
{
    __shared__ uint32_t s_ge[TT_WAVES], s_in[TT_WAVES];
    __shared__ unsigned long long s_seg[2];
    // values and positions apart: a 64-bit pair per entry made the compiler
    // hold each value in the low half of a register pair
    __shared__ uint32_t s_bits[TK_STAGE];
    __shared__ uint16_t s_loc[TK_STAGE];
    __shared__ uint32_t s_ckey[SPLIT_CAND];
    __shared__ uint16_t s_cloc[SPLIT_CAND];
    if (!w.st->ranged)
        return;
    const uint32_t lo = w.st->klo, hi = w.st->khi;
    for (int64_t tile = blockIdx.x; tile < nt; tile += gridDim.x) {
        const int64_t tile0 = tile * TK_TILE;
        const int64_t left = N - tile0;
        split_tile<DT>(x, tile, tile0, left < TK_TILE ? (uint32_t)left : (uint32_t)TK_TILE, lo, hi, w, staging,
                       s_ge, s_in, s_seg, s_bits, s_loc, s_ckey, s_cloc);
    }
}

// One workgroup of TK_REGIONS threads: the range holds T iff fewer than k
// keys lie above khi and at least k at or above klo, and nothing overflowed.
// Then the sampled path is on, and T's rank among the candidates is k minus
// the keys above khi; else the candidate counters are cleared for the full
// path.
__global__ __launch_bounds__(TK_REGIONS) void topk_check_kernel(TopkWs w, int64_t k, int g)
{
    __shared__ unsigned long long s_ge[TK_REGIONS / 64], s_in[TK_REGIONS / 64];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const unsigned long long c = w.rcnt[t * TK_CSTRIDE];
    unsigned long long ge = c >> 32, in = c & 0xFFFFFFFFull;
    for (int d = 32; d > 0; d >>= 1) {
        ge += __shfl_down(ge, d, 64);
        in += __shfl_down(in, d, 64);
    }
    if (lane == 0) {
        s_ge[wave] = ge;
        s_in[wave] = in;
    }
    const bool ranged = w.st->ranged != 0u, fov = w.st->fov != 0u;
    __syncthreads();
    unsigned long long n_ge = 0, n_in = 0;
#pragma unroll
    for (int v = 0; v < TK_REGIONS / 64; ++v) {
        n_ge += s_ge[v];
        n_in += s_in[v];
    }
    const int64_t above = (int64_t)(n_ge - n_in);
    const bool fast = ranged && !fov && above < k && k <= (int64_t)n_ge;
    // T's digits are then taken from d = (key - klo) >> g (g = 16 for bf16,
    // whose keys have zeros below bit 16) in two passes of at most 11 bits
    // when the range spans fewer than 2^22 values of d; a wider range (no
    // upper bound, for a small k) takes the candidates' absolute digits
    const uint32_t span = (w.st->khi - w.st->klo) >> g;
    const int B = span ? 32 - __clz(span) : 0;
    if (!fast)
        w.rcnt[t * TK_CSTRIDE] = 0ull;
    if (t == 0) {
        w.st->fast = fast;
        if (fast) {
            w.st->rank = k - above;
            w.st->rel = B <= 22;
            w.st->g = (uint32_t)g;
            w.st->sh1 = B > 11 ? (uint32_t)(B - 11) : 0u;
            w.st->dprefix = 0u;
        }
    }
}

// ------------------------------------------------------------ full path

// Per tile, once the top digit b1 of T is known: count the keys above bin
// b1 and compact the keys inside it into the tile's candidate segment.
template <int DT>
__global__ __launch_bounds__(TT_THREADS) void topk_split_bin_kernel(const void *x, int64_t N,
                                                                    bool vec_ok, int64_t nt, TopkWs w)
{
    __shared__ uint32_t s_wave[TT_WAVES];
    __shared__ unsigned long long s_off;
    using TL = Tile<DT>;
    if (w.st->fast)
        return;
    const uint32_t b1 = w.st->prefix >> TK_TOP_SHIFT;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int64_t tile = blockIdx.x; tile < nt; tile += gridDim.x) {
        const int64_t tile0 = tile * TK_TILE;
        TL tl;
        tl.load(x, N, vec_ok, tile0);
        uint32_t v = 0; // (keys above bin b1) << 16 | (keys inside it)
#pragma unroll
        for (int j = 0; j < TL::ROUNDS; ++j)
#pragma unroll
            for (int q = 0; q < TL::V; ++q) {
                const uint32_t bin = key_of_bits(tl.b[j][q]) >> TK_TOP_SHIFT;
                v += bin > b1 ? (1u << 16) : 0u;
                v += bin == b1 ? 1u : 0u;
            }
        const uint32_t inc = wave_inclusive_scan(v);
        if (lane == 63)
            s_wave[wave] = inc;
        __syncthreads();
        uint32_t before = 0, tot = 0;
#pragma unroll
        for (int u = 0; u < TT_WAVES; ++u) {
            before += u < wave ? s_wave[u] : 0u;
            tot += s_wave[u];
        }
        // padding (key 0) lies in bin b1 only when b1 is 0, never above it
        const uint32_t tot_def = tot >> 16, tot_cand = (tot & 0xFFFFu) - (b1 == 0u ? tl.pad() : 0u);
        if (threadIdx.x == 0) {
            const int region = (int)(tile % TK_REGIONS);
            const unsigned long long o = tot_cand ? atomicAdd(&w.rcnt[region * TK_CSTRIDE], (unsigned long long)tot_cand) : 0ull;
            const bool fits = (int64_t)(o + tot_cand) <= w.rcap;
            if (!fits)
                w.st->overflow = 1u;
            s_off = fits ? (unsigned long long)region * w.rcap + o : ~0ull;
            w.def[tile] = tot_def;
            w.ccnt[tile] = tot_cand;
            w.coff[tile] = (unsigned long long)region * w.rcap + o;
        }
        __syncthreads();
        const unsigned long long o = s_off;
        tl.reuse();
        if (o != ~0ull && (v & 0xFFFFu)) {
            uint32_t rank = (before + inc - v) & 0xFFFFu;
#pragma unroll
            for (int j = 0; j < TL::ROUNDS; ++j)
#pragma unroll
                for (int q = 0; q < TL::V; ++q) {
                    const uint32_t key = key_of_bits(tl.b[j][q]);
                    if ((key >> TK_TOP_SHIFT) == b1) {
                        if (rank < tot_cand) // padding ranks last
                            w.cand[o + rank] = u32x2{key, tl.local(j, q)};
                        ++rank;
                    }
                }
        }
        __syncthreads(); // s_wave and s_off are reused by the next tile
    }
}

// ------------------------------------------------------------ both paths

// LDS histogram of one digit, added to the global histogram once per
// workgroup.  Absolute digits: digit (key >> shift) & (bins-1) of the keys
// whose bits above it equal the prefix -- on the full path over the whole
// input for the first digit (pass 1) and over the candidates after it unless
// they overflowed, on the sampled path over the candidates.  Relative digits
// (sampled path, narrow range), over the candidates: pass 1 the upper digit
// d >> sh1 of d = (key - klo) >> g, pass 2 the lower sh1 bits of the
// candidates whose upper digit is dprefix; pass 3 has nothing to do.  The
// grid is a multiple of TK_REGIONS: gridDim / TK_REGIONS workgroups share
// each candidate region.
template <int DT>
__global__ __launch_bounds__(TK_THREADS) void topk_hist_kernel(const void *x, int64_t N,
                                                               bool vec_ok, TopkWs w, int pass,
                                                               int shift, int bits)
{
    __shared__ uint32_t s_hist[TK_WAVES][TK_MAX_BINS];
    const bool fast = w.st->fast != 0u;
    const bool rel = fast && w.st->rel != 0u;
    if (rel && pass == 3)
        return;
    const int bins = rel ? TK_MAX_BINS : 1 << bits;
    const uint32_t above =
        (shift + bits >= 31) ? 0u : (0x7FFFFFFFu >> (shift + bits)) << (shift + bits);
    const uint32_t prefix = w.st->prefix & above;
    const uint32_t klo = w.st->klo, g = w.st->g, sh1 = w.st->sh1, dprefix = w.st->dprefix;
    const bool input = !fast && (pass == 1 || w.st->overflow);
    const int wave = threadIdx.x >> 6;
    for (int b = threadIdx.x; b < TK_WAVES * bins; b += blockDim.x)
        s_hist[b / bins][b % bins] = 0u;
    __syncthreads();

    uint32_t *h = s_hist[wave];
    auto count = [&](uint32_t key) {
        if (rel) {
            const uint32_t d = (key - klo) >> g;
            if (pass == 1)
                atomicAdd(&h[d >> sh1], 1u);
            else if ((d >> sh1) == dprefix)
                atomicAdd(&h[d & ((1u << sh1) - 1u)], 1u);
        } else if ((key & above) == prefix) {
            atomicAdd(&h[(key >> shift) & (uint32_t)(bins - 1)], 1u);
        }
    };
    // the loops issue HU loads before counting any of them, so a thread
    // waits for one round trip per HU elements rather than per element
    constexpr int HU = 8;
    if (input) {
        constexpr int V = Vec<DT>::N;
        const int64_t stride = (int64_t)gridDim.x * blockDim.x;
        const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
        const int64_t nvec = vec_ok ? N / V : 0;
        int64_t v = t0;
        for (; v + (HU / 2 - 1) * stride < nvec; v += (HU / 2) * stride) {
            uint32_t b[HU / 2][V];
#pragma unroll
            for (int u = 0; u < HU / 2; ++u)
                Vec<DT>::load(x, v + u * stride, b[u]);
#pragma unroll
            for (int u = 0; u < HU / 2; ++u)
#pragma unroll
                for (int q = 0; q < V; ++q)
                    count(key_of_bits(b[u][q]));
        }
        for (; v < nvec; v += stride) {
            uint32_t b[V];
            Vec<DT>::load(x, v, b);
#pragma unroll
            for (int q = 0; q < V; ++q)
                count(key_of_bits(b[q]));
        }
        for (int64_t e = nvec * V + t0; e < N; e += stride)
            count(key_of_bits(bits_at<DT>(x, e)));
    } else {
        const int r = (int)(blockIdx.x % TK_REGIONS);
        const int64_t parts = gridDim.x / TK_REGIONS, part = blockIdx.x / TK_REGIONS;
        const int64_t n = min((int64_t)(w.rcnt[r * TK_CSTRIDE] & 0xFFFFFFFFull), w.rcap);
        const u32x2 *c = w.cand + (int64_t)r * w.rcap;
        const int64_t step = parts * blockDim.x;
        int64_t i = part * blockDim.x + threadIdx.x;
        for (; i + (HU - 1) * step < n; i += HU * step) {
            uint32_t kk[HU];
#pragma unroll
            for (int u = 0; u < HU; ++u)
                kk[u] = c[i + u * step].x;
#pragma unroll
            for (int u = 0; u < HU; ++u)
                count(kk[u]);
        }
        for (; i < n; i += step)
            count(c[i].x);
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

// One workgroup: the digit holding the rank-th key is chosen, the rank drops
// to the rank inside it, and the histogram is cleared for the next pass.
// Absolute digits: the digit joins the prefix at `shift`.  Relative digits:
// pass 1 keeps the upper digit, pass 2 completes T = klo + (((dprefix <<
// sh1) | digit) << g); pass 3 has nothing to do.
__global__ __launch_bounds__(TK_SELECT_THREADS) void topk_select_kernel(TopkWs w, int pass, int shift,
                                                                        int bits)
{
    __shared__ unsigned long long s_wtot[TK_SELECT_THREADS / 64];
    __shared__ int s_bin;
    __shared__ int64_t s_rem;
    TopkState *st = w.st;
    const bool rel = st->fast != 0u && st->rel != 0u;
    if (rel && pass == 3)
        return;
    const int bins = rel ? TK_MAX_BINS : 1 << bits;
    // read before the first barrier: thread 0 rewrites them at the end
    const int64_t rank = st->rank;
    const uint32_t dprefix = st->dprefix;
    int64_t rem;
    const int b = select_bin(w.hist, bins, rank, &rem, s_wtot, &s_bin, &s_rem);
    if (threadIdx.x == 0 && b >= 0) {
        if (!rel)
            st->prefix |= (uint32_t)b << shift;
        else if (pass == 1)
            st->dprefix = (uint32_t)b;
        else
            st->prefix = st->klo + ((((dprefix << st->sh1) | (uint32_t)b)) << st->g);
        st->rank = rem;
    }
    for (int u = threadIdx.x; u < bins; u += blockDim.x)
        w.hist[u] = 0ull;
}

// Per tile: keys above and equal to T from the tile's candidates, plus its
// keys above them.  Each wave takes TC_TPW tiles and issues their first
// loads together.  Skipped after a candidate overflow on the full path
// (topk_tile_count_input_kernel counts then).
constexpr int TC_TPW = 4;

__device__ __forceinline__ uint32_t above_or_tie(uint32_t key, uint32_t T)
{
    return key > T ? (1u << 16) : (key == T ? 1u : 0u);
}

__global__ __launch_bounds__(TT_THREADS) void topk_tile_count_kernel(int64_t nt, TopkWs w)
{
    if (!w.st->fast && w.st->overflow)
        return;
    const int64_t tile0 = ((int64_t)blockIdx.x * TT_WAVES + (threadIdx.x >> 6)) * TC_TPW;
    if (tile0 >= nt)
        return; // no barriers below
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t T = w.st->prefix;
    uint32_t n[TC_TPW], c[TC_TPW];
    unsigned long long c0[TC_TPW];
#pragma unroll
    for (int i = 0; i < TC_TPW; ++i) {
        const bool ok = tile0 + i < nt;
        n[i] = ok ? w.ccnt[tile0 + i] : 0u;
        c0[i] = ok ? w.coff[tile0 + i] : 0ull;
    }
#pragma unroll
    for (int i = 0; i < TC_TPW; ++i)
        c[i] = lane < n[i] ? above_or_tie(w.cand[c0[i] + lane].x, T) : 0u;
#pragma unroll
    for (int i = 0; i < TC_TPW; ++i)
        for (uint32_t j = lane + 64; j < n[i]; j += 64)
            c[i] += above_or_tie(w.cand[c0[i] + j].x, T);
    // each below 2^16 per tile, so the packed sums never carry
#pragma unroll
    for (int i = 0; i < TC_TPW; ++i) {
        const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_scan(c[i]), 63);
        if (lane == 0 && tile0 + i < nt) {
            w.gt[tile0 + i] = (tot >> 16) + w.def[tile0 + i];
            w.eq[tile0 + i] = tot & 0xFFFFu;
        }
    }
}

// The same counts from the whole tile, after a candidate overflow on the
// full path.
template <int DT>
__global__ __launch_bounds__(TT_THREADS) void topk_tile_count_input_kernel(const void *x, int64_t N,
                                                                           bool vec_ok, int64_t nt,
                                                                           TopkWs w)
{
    __shared__ uint32_t s_sum[TT_WAVES];
    if (w.st->fast || !w.st->overflow)
        return;
    using TL = Tile<DT>;
    const uint32_t T = w.st->prefix;
    for (int64_t tile = blockIdx.x; tile < nt; tile += gridDim.x) {
        const int64_t tile0 = tile * TK_TILE;
        TL tl;
        tl.load(x, N, vec_ok, tile0);
        uint32_t c = 0;
#pragma unroll
        for (int j = 0; j < TL::ROUNDS; ++j)
#pragma unroll
            for (int q = 0; q < TL::V; ++q) {
                const uint32_t key = key_of_bits(tl.b[j][q]);
                c += key > T ? (1u << 16) : 0u;
                c += key == T ? 1u : 0u;
            }
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
            w.gt[tile] = s >> 16;
            w.eq[tile] = (s & 0xFFFFu) - (T == 0u ? tl.pad() : 0u); // padding is key 0
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------ offsets

// Tile b keeps take[b] = clamp(r - ties before b, 0, eq[b]) of its ties and
// writes from off[b] = sum over earlier tiles of gt + take.  Three kernels:
// per chunk of TK_SCAN_CHUNK tiles the sums of eq and gt; one workgroup over
// the chunks; then each chunk's tiles.

// Four tiles' counts from b0 (the arrays are padded to a multiple of 4).
__device__ __forceinline__ void load4(const uint32_t *a, int64_t b0, int64_t nt, uint32_t o[4])
{
    o[0] = o[1] = o[2] = o[3] = 0u;
    if (b0 < nt) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(a + b0);
        const int64_t live = nt - b0;
        o[0] = v.x;
        o[1] = live > 1 ? v.y : 0u;
        o[2] = live > 2 ? v.z : 0u;
        o[3] = live > 3 ? v.w : 0u;
    }
}

__global__ __launch_bounds__(256) void topk_scan_reduce_kernel(int64_t nt, TopkWs w)
{
    __shared__ int64_t s_tmp[256 / 64 + 1];
    const int64_t b0 = (int64_t)blockIdx.x * TK_SCAN_CHUNK + 4 * (int64_t)threadIdx.x;
    uint32_t g[4], e[4];
    load4(w.gt, b0, nt, g);
    load4(w.eq, b0, nt, e);
    int64_t tot_e, tot_g;
    block_exclusive_scan64<256>((int64_t)e[0] + e[1] + e[2] + e[3], s_tmp, tot_e);
    block_exclusive_scan64<256>((int64_t)g[0] + g[1] + g[2] + g[3], s_tmp, tot_g);
    if (threadIdx.x == 0) {
        w.ch_eq[blockIdx.x] = tot_e;
        w.ch_gt[blockIdx.x] = tot_g;
    }
}

__global__ __launch_bounds__(TK_SELECT_THREADS) void topk_scan_top_kernel(int64_t nch, TopkWs w)
{
    __shared__ int64_t s_tmp[TK_SELECT_THREADS / 64 + 1];
    const int64_t r = w.st->rank;
    int64_t ties_carry = 0, sel_carry = 0;
    for (int64_t c0 = 0; c0 < nch; c0 += TK_SELECT_THREADS) {
        const int64_t c = c0 + threadIdx.x;
        const int64_t e = c < nch ? w.ch_eq[c] : 0, g = c < nch ? w.ch_gt[c] : 0;
        int64_t total;
        const int64_t tb = ties_carry + block_exclusive_scan64<TK_SELECT_THREADS>(e, s_tmp, total);
        ties_carry += total;
        const int64_t sel = g + max((int64_t)0, min(r - tb, e));
        const int64_t ob = sel_carry + block_exclusive_scan64<TK_SELECT_THREADS>(sel, s_tmp, total);
        sel_carry += total;
        if (c < nch) {
            w.ch_ties[c] = tb;
            w.ch_off[c] = ob;
        }
    }
}

__global__ __launch_bounds__(256) void topk_scan_down_kernel(int64_t nt, TopkWs w)
{
    __shared__ int64_t s_tmp[256 / 64 + 1];
    const int64_t r = w.st->rank;
    const int64_t b0 = (int64_t)blockIdx.x * TK_SCAN_CHUNK + 4 * (int64_t)threadIdx.x;
    uint32_t g[4], e[4];
    load4(w.gt, b0, nt, g);
    load4(w.eq, b0, nt, e);
    int64_t total;
    int64_t tb = w.ch_ties[blockIdx.x] +
                 block_exclusive_scan64<256>((int64_t)e[0] + e[1] + e[2] + e[3], s_tmp, total);
    uint32_t tk[4];
    int64_t sel = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        tk[i] = (uint32_t)max((int64_t)0, min(r - tb, (int64_t)e[i]));
        tb += e[i];
        sel += g[i] + tk[i];
    }
    int64_t ob = w.ch_off[blockIdx.x] + block_exclusive_scan64<256>(sel, s_tmp, total);
    const int live = b0 < nt ? (int)min((int64_t)4, nt - b0) : 0;
    for (int i = 0; i < live; ++i) {
        w.take[b0 + i] = tk[i];
        w.off[b0 + i] = ob;
        ob += g[i] + tk[i];
    }
}

// ------------------------------------------------------------ the write

// Sampled path with staging: each tile's kept entries from its staging
// segment (already in index order), in chunks of TW_ROUNDS x TW_THREADS
// entries; every round's entries get their rank among the kept ones from wave
// scans of the packed (above, tie) counts and one exchange of per-wave totals
// in LDS.  Small workgroups with many entries per thread keep more tiles,
// and so more loads, in flight per CU.
constexpr int TW_THREADS = 128;
constexpr int TW_TILES = 2; // tiles a workgroup of the staged write takes at once
constexpr int TW_WAVES = TW_THREADS / 64;
constexpr int TW_ROUNDS = 8;

// One chunk of up to TW_ROUNDS * TW_THREADS staged entries of a tile,
// loaded (ent, entries at or past n read as key 0), ranked and written.
// `carry` holds the packed counts of the tile's entries before the chunk.
template <int DT>
__device__ __forceinline__ void write_staged_chunk(const u32x2 (&ent)[TW_ROUNDS], uint32_t c0, uint32_t n,
                                                   uint32_t T, uint32_t tk, int64_t base, int64_t tile0,
                                                   int64_t k_out, int64_t *idx_out, float *val_out,
                                                   uint32_t (*s_tot)[TW_WAVES], uint32_t &carry)
{
    constexpr int R = TW_ROUNDS;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t exw[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const uint32_t p = c0 + i * TW_THREADS + threadIdx.x;
        const uint32_t key = key_of_bits(ent[i].x);
        const uint32_t v = p < n ? (key > T ? (1u << 16) : (key == T ? 1u : 0u)) : 0u;
        const uint32_t sc = wave_inclusive_scan(v);
        if (lane == 63)
            s_tot[i][wave] = sc;
        exw[i] = sc - v;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < R; ++i) {
        uint32_t before = 0, round_total = 0;
#pragma unroll
        for (int v = 0; v < TW_WAVES; ++v) {
            const uint32_t t = s_tot[i][v];
            before += v < wave ? t : 0u;
            round_total += t;
        }
        const uint32_t run = carry + before + exw[i];
        carry += round_total;
        const uint32_t p = c0 + i * TW_THREADS + threadIdx.x;
        const uint32_t key = key_of_bits(ent[i].x);
        if (p >= n || key < T)
            continue;
        const uint32_t gt_before = run >> 16, eq_before = run & 0xFFFFu;
        if (key == T && eq_before >= tk)
            continue;
        const int64_t r = base + gt_before + min(eq_before, tk);
        if (r < k_out) { // keeps inconsistent counts from writing out of range
            idx_out[r] = tile0 + ent[i].y;
            val_out[r] = __uint_as_float(ent[i].x);
        }
    }
    __syncthreads(); // s_tot is reused by the next chunk
}

template <int DT>
__device__ __forceinline__ void load_staged_chunk(const TopkWs &w, uint64_t seg, uint32_t c0, uint32_t n,
                                                  u32x2 (&ent)[TW_ROUNDS])
{
#pragma unroll
    for (int i = 0; i < TW_ROUNDS; ++i) {
        const uint32_t p = c0 + i * TW_THREADS + threadIdx.x;
        ent[i] = p < n ? u32x2{stage_bits<DT>(w, seg + p), (uint32_t)w.sloc[seg + p]} : u32x2{0u, 0u};
    }
}

// Each workgroup writes TW_TILES consecutive tiles: the first chunks of all
// of them are loaded before any is ranked, so a workgroup has that many
// tiles' entries in flight at once.
template <int DT>
__global__ __launch_bounds__(TW_THREADS) void topk_write_staged_kernel(int64_t nt, TopkWs w,
                                                                       int64_t k_out,
                                                                       int64_t *idx_out,
                                                                       float *val_out)
{
    constexpr int CH = TW_ROUNDS * TW_THREADS;
    __shared__ uint32_t s_tot[TW_ROUNDS][TW_WAVES];
    if (!w.st->fast)
        return;
    const uint32_t T = w.st->prefix;
    for (int64_t t0 = (int64_t)blockIdx.x * TW_TILES; t0 < nt; t0 += (int64_t)gridDim.x * TW_TILES) {
        uint32_t n[TW_TILES], tk[TW_TILES];
        uint64_t seg[TW_TILES];
        int64_t base[TW_TILES];
        u32x2 ent[TW_TILES][TW_ROUNDS];
#pragma unroll
        for (int u = 0; u < TW_TILES; ++u) {
            const bool has = t0 + u < nt;
            n[u] = has ? w.tcnt[t0 + u] : 0u;
            seg[u] = has ? w.toff[t0 + u] : 0ull;
            tk[u] = has ? w.take[t0 + u] : 0u;
            base[u] = has ? w.off[t0 + u] : 0;
        }
#pragma unroll
        for (int u = 0; u < TW_TILES; ++u)
            load_staged_chunk<DT>(w, seg[u], 0, n[u], ent[u]);
#pragma unroll
        for (int u = 0; u < TW_TILES; ++u) {
            const int64_t tile0 = (t0 + u) * TK_TILE;
            uint32_t carry = 0; // packed counts of the entries before this chunk
            write_staged_chunk<DT>(ent[u], 0, n[u], T, tk[u], base[u], tile0, k_out, idx_out, val_out, s_tot,
                                   carry);
            // a tile keeping more than CH entries (over an eighth of it)
            for (uint32_t c0 = CH; c0 < n[u]; c0 += CH) {
                u32x2 more[TW_ROUNDS];
                load_staged_chunk<DT>(w, seg[u], c0, n[u], more);
                write_staged_chunk<DT>(more, c0, n[u], T, tk[u], base[u], tile0, k_out, idx_out, val_out,
                                       s_tot, carry);
            }
        }
    }
}

// From the update itself (full path, or the sampled path without staging):
// the tile is loaded whole into registers and ranked as above; the first
// TK_STAGE kept entries are staged in LDS and written out as two contiguous
// runs, any beyond that (a tile keeping more than a quarter of its elements)
// go straight out.
template <int DT>
__global__ __launch_bounds__(TT_THREADS) void topk_write_input_kernel(const void *x, int64_t N,
                                                                      bool vec_ok, int64_t nt,
                                                                      TopkWs w, bool staged,
                                                                      int64_t k_out, int64_t *idx_out,
                                                                      float *val_out)
{
    using TL = Tile<DT>;
    __shared__ uint32_t s_tot[TL::ROUNDS][TT_WAVES];
    __shared__ uint32_t s_idx[TK_STAGE];
    __shared__ float s_val[TK_STAGE];
    if (staged && w.st->fast)
        return;
    const uint32_t T = w.st->prefix;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int64_t tile = blockIdx.x; tile < nt; tile += gridDim.x) {
        const int64_t tile0 = tile * TK_TILE;
        const uint32_t tk = w.take[tile];
        const int64_t base = w.off[tile];
        TL tl;
        tl.load(x, N, vec_ok, tile0);
        uint32_t exw[TL::ROUNDS];
#pragma unroll
        for (int j = 0; j < TL::ROUNDS; ++j) {
            uint32_t v = 0;
#pragma unroll
            for (int q = 0; q < TL::V; ++q) {
                const uint32_t key = key_of_bits(tl.b[j][q]);
                v += key > T ? (1u << 16) : 0u;
                v += key == T ? 1u : 0u;
            }
            const uint32_t sc = wave_inclusive_scan(v);
            if (lane == 63)
                s_tot[j][wave] = sc;
            exw[j] = sc - v; // this lane's exclusive prefix inside its wave
        }
        __syncthreads();
        tl.reuse();
        uint32_t carry = 0; // packed counts of the rounds before j
#pragma unroll
        for (int j = 0; j < TL::ROUNDS; ++j) {
            uint32_t before = 0, round_total = 0;
#pragma unroll
            for (int v = 0; v < TT_WAVES; ++v) {
                const uint32_t t = s_tot[j][v];
                before += v < wave ? t : 0u;
                round_total += t;
            }
            const uint32_t run = carry + before + exw[j];
            carry += round_total;
            uint32_t gt_before = run >> 16, eq_before = run & 0xFFFFu;
#pragma unroll
            for (int q = 0; q < TL::V; ++q) {
                const uint32_t bits = tl.b[j][q];
                const uint32_t key = key_of_bits(bits);
                // padding (key 0) is never above T, and as a tie it ranks
                // after the tile's own ties, of which at most tk are kept
                if (key < T)
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
                const uint32_t local = tl.local(j, q);
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
        const uint32_t kept_total = (carry >> 16) + min(carry & 0xFFFFu, tk);
        __syncthreads();
        const int n = (int)min((uint32_t)TK_STAGE, kept_total);
        for (int i = threadIdx.x; i < n; i += TT_THREADS) {
            if (base + i < k_out) {
                idx_out[base + i] = tile0 + s_idx[i];
                val_out[base + i] = s_val[i];
            }
        }
        __syncthreads(); // s_tot and the staging arrays are reused by the next tile
    }
}

unsigned grid_of(int64_t work, int64_t cap)
{
    int64_t g = (work + TK_THREADS - 1) / TK_THREADS;
    if (g > cap)
        g = cap;
    return (unsigned)(g < 1 ? 1 : g);
}

int g_topk_sampled = 1; // FA_OPT_TOPK_SAMPLED

// The sample and the two order statistics that bound T.  m keys are
// sampled; T has expected rank rho = k m / N among them (from the top) with
// binomial standard deviation sigma = sqrt(rho (1 - k/N)); K_hi comes from
// the sample's r_hi-th largest key, r_hi = floor(rho - 8 sigma - 32) (no
// upper bound when r_hi < 1), and K_lo from its r_lo-th, r_lo = ceil(rho +
// 8 sigma + 32) (no sampled path when r_lo > m).
struct SamplePlan {
    bool on, has_hi, vec_units;
    int64_t units, mu, r_hi, r_lo;
};

template <int DT> SamplePlan plan_sample(int64_t N, int64_t k, bool vec_ok)
{
    SamplePlan p = {};
    p.vec_units = vec_ok;
    const int64_t width = vec_ok ? Vec<DT>::N : 1;
    p.units = vec_ok ? N / Vec<DT>::N : N;
    const int64_t cap = TK_SAMPLE_KEYS / width;
    p.mu = p.units < cap ? p.units : cap;
    if (!g_topk_sampled || p.mu < 1 || k >= N)
        return p;
    const double m = (double)(p.mu * width);
    const double rho = (double)k * m / (double)N;
    const double sigma = sqrt(rho * (1.0 - (double)k / (double)N));
    const double margin = 8.0 * sigma + 32.0;
    p.r_hi = (int64_t)floor(rho - margin);
    p.has_hi = p.r_hi >= 1;
    p.r_lo = (int64_t)ceil(rho + margin);
    p.on = p.r_lo <= p.mu * width;
    return p;
}

template <int DT>
hipError_t topk_run(const void *x, int64_t N, int64_t k, int64_t *idx_out, float *val_out,
                    void *ws, int cus, hipStream_t s)
{
    const Sizes sz = sizes_of(N, k, DT);
    const TopkWs w = carve(ws, sz, DT);
    const int64_t nt = sz.nt;
    const bool vec_ok = (reinterpret_cast<uintptr_t>(x) & 15u) == 0;
    const bool staging = sz.tcap > 0;
    const SamplePlan plan = plan_sample<DT>(N, k, vec_ok);
    const unsigned full_grid = grid_of(N / Vec<DT>::N + 1, (int64_t)cus * 4);
    // a multiple of TK_REGIONS, so every candidate region gets the same share
    const unsigned hist_grid = (full_grid + TK_REGIONS - 1) / TK_REGIONS * TK_REGIONS;
    // Per-tile kernels loop over tiles, so any grid is correct.  One that
    // will most likely do the work gets a workgroup per tile (the dispatcher
    // then overlaps the phases of many tiles per CU); one that most likely
    // finds its path off and exits gets a small grid.
    const unsigned work_grid = (unsigned)nt;
    const int64_t idle_cap = (int64_t)cus * 2;
    const unsigned idle_grid = (unsigned)(nt < idle_cap ? nt : idle_cap);

    topk_init_kernel<<<1, 256, 0, s>>>(w, k);
    if (plan.on) {
        const unsigned sg = grid_of(plan.mu, 256);
        topk_sample_hist_kernel<DT><<<sg, TK_THREADS, 0, s>>>(x, plan.vec_units, plan.units, plan.mu, w, 1, plan.has_hi);
        topk_sample_select_kernel<<<1, TK_SELECT_THREADS, 0, s>>>(w, 1, plan.has_hi, plan.r_hi, plan.r_lo);
        topk_sample_hist_kernel<DT><<<sg, TK_THREADS, 0, s>>>(x, plan.vec_units, plan.units, plan.mu, w, 2, plan.has_hi);
        topk_sample_select_kernel<<<1, TK_SELECT_THREADS, 0, s>>>(w, 2, plan.has_hi, plan.r_hi, plan.r_lo);
        topk_split_range_kernel<DT><<<work_grid, TT_THREADS, 0, s>>>(x, N, nt, w, staging);
        topk_check_kernel<<<1, TK_REGIONS, 0, s>>>(w, k, DT == DT_BF16 ? 16 : 0);
    }
    // Full path: digit 1 (key bits 30..20) from the whole input, the split,
    // then digits 2 (bits 19..9) and, for fp32, 3 (bits 8..0) from the
    // candidates; a bf16 key has zeros below bit 16, so two digits decide it.
    // Sampled path: the same digits from the candidates, or for a narrow
    // range two digits of (key - klo) >> g and the third pair of launches
    // exits.
    topk_hist_kernel<DT><<<hist_grid, TK_THREADS, 0, s>>>(x, N, vec_ok, w, 1, TK_TOP_SHIFT, 11);
    topk_select_kernel<<<1, TK_SELECT_THREADS, 0, s>>>(w, 1, TK_TOP_SHIFT, 11);
    topk_split_bin_kernel<DT><<<plan.on ? idle_grid : work_grid, TT_THREADS, 0, s>>>(x, N, vec_ok, nt, w);
    topk_hist_kernel<DT><<<hist_grid, TK_THREADS, 0, s>>>(x, N, vec_ok, w, 2, TK_SUB_SHIFT, 11);
    topk_select_kernel<<<1, TK_SELECT_THREADS, 0, s>>>(w, 2, TK_SUB_SHIFT, 11);
    if (DT == DT_F32) {
        topk_hist_kernel<DT><<<hist_grid, TK_THREADS, 0, s>>>(x, N, vec_ok, w, 3, 0, 9);
        topk_select_kernel<<<1, TK_SELECT_THREADS, 0, s>>>(w, 3, 0, 9);
    }
    topk_tile_count_kernel<<<(unsigned)((nt + TT_WAVES * TC_TPW - 1) / (TT_WAVES * TC_TPW)), TT_THREADS, 0, s>>>(nt, w);
    topk_tile_count_input_kernel<DT><<<idle_grid, TT_THREADS, 0, s>>>(x, N, vec_ok, nt, w);
    topk_scan_reduce_kernel<<<(unsigned)sz.nch, 256, 0, s>>>(nt, w);
    topk_scan_top_kernel<<<1, TK_SELECT_THREADS, 0, s>>>(sz.nch, w);
    topk_scan_down_kernel<<<(unsigned)sz.nch, 256, 0, s>>>(nt, w);
    const bool staged = plan.on && staging;
    if (staged)
        topk_write_staged_kernel<DT><<<(unsigned)((nt + TW_TILES - 1) / TW_TILES), TW_THREADS, 0, s>>>(
            nt, w, k, idx_out, val_out);
    topk_write_input_kernel<DT><<<staged ? idle_grid : work_grid, TT_THREADS, 0, s>>>(x, N, vec_ok, nt, w, staged, k, idx_out, val_out);
    return hipGetLastError();
}

} // namespace

size_t topk_workspace_bytes(int dt, int64_t N, int64_t k) { return sizes_of(N, k, dt).bytes; }

void topk_set_sampled(int on) { g_topk_sampled = on; }

hipError_t launch_topk(const void *x, int dt, int64_t N, int64_t k, int64_t *idx_out,
                       float *val_out, void *ws, int cus, hipStream_t s)
{
    return dt == DT_F32 ? topk_run<DT_F32>(x, N, k, idx_out, val_out, ws, cus, s)
                        : topk_run<DT_BF16>(x, N, k, idx_out, val_out, ws, cus, s);
}

} // namespace fa
