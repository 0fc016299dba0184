// HBM ceilings of the aggregation kernels' byte patterns on gfx950, for the
// benchmark only (libhbm_ceiling.so; the aggregation library never loads it).
//
// Each kernel moves the bytes of one aggregation pattern with no arithmetic
// beyond an XOR that keeps the loads live:
//   read   NS streams read, nothing written (a store that never fires keeps
//          the loads alive);
//   mix    NS streams read and one written, 16 bytes per 16 bytes of each
//          input -- the resident dense aggregation's pattern (16 clients in,
//          one output) without its FMAs;
//   copy   the mix with one input.
// The cache policy of the loads and of the stores is a template argument:
// plain or non-temporal global accesses, or buffer accesses carrying any of
// the sc0 / sc1 / nt bits.  VPT vectors per thread are loaded and combined one
// after another and their results stored together at the end (write
// batching).  The grid strides over the vectors; residency per CU is capped,
// when asked, by reserving dynamic LDS the kernel does not use.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Policies: how a load or a store reaches memory.
enum Pol {
    P_GLOBAL = 0,      // global access, no cache bits
    P_GLOBAL_NT = 1,   // global access, nt
    P_BUF = 2,         // buffer access, no cache bits
    P_BUF_NT = 3,      // buffer, nt
    P_BUF_SC1 = 4,     // buffer, sc1 (device scope)
    P_BUF_SC0SC1 = 5,  // buffer, sc0 sc1 (system scope)
    P_BUF_SC1NT = 6,   // buffer, sc1 nt
    P_BUF_SC0SC1NT = 7 // buffer, sc0 sc1 nt
};

// buffer instruction cache-policy immediate: bit 0 sc0, bit 1 nt, bit 4 sc1
template <int P> constexpr int aux()
{
    return P == P_BUF_NT ? 2
           : P == P_BUF_SC1 ? 16
           : P == P_BUF_SC0SC1 ? 17
           : P == P_BUF_SC1NT ? 18
           : P == P_BUF_SC0SC1NT ? 19
                                  : 0;
}

// raw buffer over one stream of at most 2^32 - 1 bytes
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, 0x00020000);
}

template <int P> __device__ __forceinline__ u32x4 load16(const void *base, uint32_t bytes, int64_t v)
{
    if constexpr (P == P_GLOBAL)
        return reinterpret_cast<const u32x4 *>(base)[v];
    else if constexpr (P == P_GLOBAL_NT)
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(base) + v);
    else
        return __builtin_amdgcn_raw_buffer_load_b128(rsrc(base, bytes), (int)(v * 16), 0, aux<P>());
}

template <int P> __device__ __forceinline__ void store16(void *base, uint32_t bytes, int64_t v, u32x4 x)
{
    if constexpr (P == P_GLOBAL)
        reinterpret_cast<u32x4 *>(base)[v] = x;
    else if constexpr (P == P_GLOBAL_NT)
        __builtin_nontemporal_store(x, reinterpret_cast<u32x4 *>(base) + v);
    else
        __builtin_amdgcn_raw_buffer_store_b128(x, rsrc(base, bytes), (int)(v * 16), 0, aux<P>());
}

constexpr int MAX_STREAMS = 17;

struct HcArgs {
    const void *src[MAX_STREAMS];
    void *dst;
    int64_t nvec;   // 16-byte vectors per stream
    uint32_t bytes; // bytes per stream (buffer range)
    uint32_t magic; // the read-only kernel stores only when its XOR equals this
};

template <int NS, int LP, int SP, int VPT, bool WRITE>
__global__ __launch_bounds__(256) void stream_kernel(const HcArgs a)
{
    const int64_t stride = (int64_t)gridDim.x * 256 * VPT;
    for (int64_t v0 = (int64_t)blockIdx.x * 256 * VPT + threadIdx.x; v0 < a.nvec; v0 += stride) {
        u32x4 r[VPT];
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int64_t v = v0 + (int64_t)j * 256;
            u32x4 x[NS];
            if (v < a.nvec) {
#pragma unroll
                for (int s = 0; s < NS; ++s)
                    x[s] = load16<LP>(a.src[s], a.bytes, v);
            } else {
#pragma unroll
                for (int s = 0; s < NS; ++s)
                    x[s] = u32x4{0u, 0u, 0u, 0u};
            }
            u32x4 acc = x[0];
#pragma unroll
            for (int s = 1; s < NS; ++s)
                acc ^= x[s];
            r[j] = acc;
        }
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int64_t v = v0 + (int64_t)j * 256;
            if (v < a.nvec && (WRITE || r[j].x == a.magic))
                store16<SP>(a.dst, a.bytes, v, r[j]);
        }
    }
}

int lds_per_cu()
{
    static std::atomic<int> cache{0};
    int v = cache.load(std::memory_order_relaxed);
    if (v == 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
                hipSuccess ||
            v <= 0)
            v = 65536;
        cache.store(v, std::memory_order_relaxed);
    }
    return v;
}

template <typename F> size_t residency_lds(F *kernel, int cap)
{
    if (cap <= 0)
        return 0;
    const int lds = lds_per_cu();
    const size_t bytes = ((size_t)lds / cap + (size_t)lds / (cap + 1)) / 2;
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return bytes;
}

template <int NS, int LP, int SP, int VPT, bool WRITE>
int run(const HcArgs &a, int64_t grid, int resident, hipStream_t s)
{
    auto *k = &stream_kernel<NS, LP, SP, VPT, WRITE>;
    k<<<(unsigned)grid, 256, residency_lds(k, resident), s>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -9;
}

} // namespace

extern "C" {

/*
 * hc_stream -- one launch of a ceiling kernel.
 * pattern 0: read ns streams; 1: read ns streams and write one.
 * src: ns device pointers of nvec 16-byte vectors each (16-byte aligned,
 * at most 2^32 - 1 bytes each); dst: nvec vectors (pattern 1), or a buffer
 * of nvec vectors the read-only kernel practically never writes.
 * lpol, spol: Pol codes.  vpt: vectors per thread before the stores (1, 2,
 * 4).  resident: workgroups of 256 per CU (0: hardware limit).  grid:
 * workgroups (0: one vector group per thread).  Returns 0, -1 for an
 * unsupported combination or arguments, -9 for a launch error.
 */
int hc_stream(int pattern, int ns, const void *const *src, void *dst, int64_t nvec, int lpol,
              int spol, int vpt, int resident, int64_t grid, void *stream)
{
    if (ns < 1 || ns > MAX_STREAMS || !src || !dst || nvec <= 0 || nvec * 16 > 0xFFFFFFFFll)
        return -1;
    HcArgs a;
    for (int s = 0; s < MAX_STREAMS; ++s)
        a.src[s] = s < ns ? src[s] : nullptr;
    a.dst = dst;
    a.nvec = nvec;
    a.bytes = (uint32_t)(nvec * 16);
    a.magic = 0x5bd1e995u;
    if (grid <= 0)
        grid = (nvec + 256 * vpt - 1) / (256 * vpt);
    if (grid > 0xFFFFFFFFll / 256)
        grid = 0xFFFFFFFFll / 256;
    hipStream_t s = static_cast<hipStream_t>(stream);
#define HC(P, N, L, S, V)                                                                          \
    if (pattern == P && ns == N && lpol == L && spol == S && vpt == V)                            \
        return run<N, L, S, V, P == 1>(a, grid, resident, s);
    // read-only, 16 and 17 streams
    HC(0, 16, P_GLOBAL_NT, P_GLOBAL, 1)
    HC(0, 16, P_GLOBAL, P_GLOBAL, 1)
    HC(0, 17, P_GLOBAL_NT, P_GLOBAL, 1)
    HC(0, 17, P_GLOBAL, P_GLOBAL, 1)
    // copy
    HC(1, 1, P_GLOBAL_NT, P_GLOBAL_NT, 1)
    HC(1, 1, P_GLOBAL, P_GLOBAL, 1)
    HC(1, 1, P_GLOBAL_NT, P_GLOBAL, 1)
    HC(1, 1, P_GLOBAL_NT, P_GLOBAL_NT, 4)
    // 16 read + 1 write: load policies with non-temporal stores
    HC(1, 16, P_GLOBAL_NT, P_GLOBAL_NT, 1)
    HC(1, 16, P_GLOBAL, P_GLOBAL_NT, 1)
    HC(1, 16, P_BUF, P_GLOBAL_NT, 1)
    HC(1, 16, P_BUF_NT, P_GLOBAL_NT, 1)
    HC(1, 16, P_BUF_SC1, P_GLOBAL_NT, 1)
    HC(1, 16, P_BUF_SC0SC1, P_GLOBAL_NT, 1)
    HC(1, 16, P_BUF_SC1NT, P_GLOBAL_NT, 1)
    // store policies with non-temporal loads
    HC(1, 16, P_GLOBAL_NT, P_GLOBAL, 1)
    HC(1, 16, P_GLOBAL_NT, P_BUF, 1)
    HC(1, 16, P_GLOBAL_NT, P_BUF_NT, 1)
    HC(1, 16, P_GLOBAL_NT, P_BUF_SC1, 1)
    HC(1, 16, P_GLOBAL_NT, P_BUF_SC0SC1, 1)
    HC(1, 16, P_GLOBAL_NT, P_BUF_SC1NT, 1)
    HC(1, 16, P_GLOBAL_NT, P_BUF_SC0SC1NT, 1)
    // buffer loads and stores (the dense kernel's accesses)
    HC(1, 16, P_BUF_NT, P_BUF_NT, 1)
    HC(1, 16, P_BUF_NT, P_BUF_SC1NT, 1)
    // fewer read streams per written one
    HC(1, 2, P_GLOBAL_NT, P_GLOBAL_NT, 1)
    HC(1, 4, P_GLOBAL_NT, P_GLOBAL_NT, 1)
    HC(1, 8, P_GLOBAL_NT, P_GLOBAL_NT, 1)
    // write batching
    HC(1, 16, P_GLOBAL_NT, P_GLOBAL_NT, 2)
    HC(1, 16, P_GLOBAL_NT, P_GLOBAL_NT, 4)
    HC(1, 16, P_GLOBAL_NT, P_GLOBAL, 2)
    HC(1, 16, P_GLOBAL_NT, P_GLOBAL, 4)
#undef HC
    return -1;
}

} // extern "C"
