// gfx950 (CDNA4) kernels of the FedAvg aggregation library.
//
// Every kernel here is bound by memory traffic (a weighted sum does one FMA
// per 2 or 4 bytes read), so the design goals are: each byte read from HBM
// once, 16-byte coalesced loads with many independent loads in flight per
// lane, non-temporal streaming stores, and no floating-point atomics (results
// must be deterministic).  There is no matrix-core work: nothing here is a
// contraction.
//
// Arithmetic order shared by all kernels, per parameter: acc = 0; for every
// contributing client in order, acc = fma(fp32(n_k), x_k, acc); q = acc /
// fp32(W) (IEEE division); in delta mode r = base + q; then
// round-to-nearest-even to the output type.  This is the fp32 weighted mean
// of the Clara page ("NVIDIA Clara implements federated learning",
// introduction and server-side workflow) with fp32 master-weight
// accumulation and nearest-even rounding of weights ("NVFP4 training with JAX
// and MaxText", training-recipe section).
#include <atomic>
#include <map>
#include <mutex>

#include "fedavg_internal.h"

namespace fa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- formats

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest, ties to even: the dropped half of the
// pattern carries into the kept half when it is above one half, or exactly
// one half with an odd kept half; a carry out of the fraction bumps the
// exponent, which turns the largest finite values into infinity.  NaN keeps
// its sign and upper payload bits and is made quiet (bit 6 set).  gfx950's
// v_cvt_pk_bf16_f32 rounds two values this way in one instruction; under the
// kernels' modes (round to nearest even, fp32 denormals kept) its result was
// compared with this definition, written as integer arithmetic on the bit
// pattern, over all 2^32 inputs, NaNs and subnormals included, with no
// difference.  The integer form took about five instructions and a branch per
// value.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

template <int DT> struct io;

template <> struct io<DT_F32> {
    struct raw {
        f32x4 a, b;
    };
    static __device__ __forceinline__ raw zero_raw() { return raw{f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}}; }
    static __device__ __forceinline__ raw load_raw(const void *p, int64_t e)
    {
        const f32x4 *q = reinterpret_cast<const f32x4 *>(static_cast<const float *>(p) + e);
        return raw{__builtin_nontemporal_load(q), __builtin_nontemporal_load(q + 1)};
    }
    static __device__ __forceinline__ void fma8(const raw &r, float w, float (&acc)[VEC])
    {
        acc[0] = __builtin_fmaf(w, r.a.x, acc[0]);
        acc[1] = __builtin_fmaf(w, r.a.y, acc[1]);
        acc[2] = __builtin_fmaf(w, r.a.z, acc[2]);
        acc[3] = __builtin_fmaf(w, r.a.w, acc[3]);
        acc[4] = __builtin_fmaf(w, r.b.x, acc[4]);
        acc[5] = __builtin_fmaf(w, r.b.y, acc[5]);
        acc[6] = __builtin_fmaf(w, r.b.z, acc[6]);
        acc[7] = __builtin_fmaf(w, r.b.w, acc[7]);
    }
    static __device__ __forceinline__ void load8(const void *p, int64_t e, float (&v)[VEC])
    {
        const f32x4 *q = reinterpret_cast<const f32x4 *>(static_cast<const float *>(p) + e);
        f32x4 a = __builtin_nontemporal_load(q);
        f32x4 b = __builtin_nontemporal_load(q + 1);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    static __device__ __forceinline__ void load4(const void *p, int64_t e, float (&v)[4])
    {
        const f32x4 a = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4 *>(static_cast<const float *>(p) + e));
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    }
    // the 8 parameters as two quads at e0 and e1 (contiguous when e1 = e0 + 4)
    static __device__ __forceinline__ raw load_raw2(const void *p, int64_t e0, int64_t e1)
    {
        const float *f = static_cast<const float *>(p);
        return raw{__builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(f + e0)),
                   __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(f + e1))};
    }
    static __device__ __forceinline__ void load8_2(const void *p, int64_t e0, int64_t e1, float (&v)[VEC])
    {
        const raw r = load_raw2(p, e0, e1);
        v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
        v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
    }
    static __device__ __forceinline__ void store8_2(void *p, int64_t e0, int64_t e1, const float (&v)[VEC])
    {
        float *f = static_cast<float *>(p);
        __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4 *>(f + e0));
        __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, reinterpret_cast<f32x4 *>(f + e1));
    }
    static __device__ __forceinline__ float load1(const void *p, int64_t e)
    {
        return static_cast<const float *>(p)[e];
    }
    static __device__ __forceinline__ void store8(void *p, int64_t e, const float (&v)[VEC])
    {
        f32x4 *q = reinterpret_cast<f32x4 *>(static_cast<float *>(p) + e);
        f32x4 a = {v[0], v[1], v[2], v[3]};
        f32x4 b = {v[4], v[5], v[6], v[7]};
        __builtin_nontemporal_store(a, q);
        __builtin_nontemporal_store(b, q + 1);
    }
    static __device__ __forceinline__ void store1(void *p, int64_t e, float v)
    {
        static_cast<float *>(p)[e] = v;
    }
};

template <> struct io<DT_BF16> {
    // eight bf16 kept packed until they are used
    struct raw {
        u32x4 v;
    };
    static __device__ __forceinline__ raw zero_raw() { return raw{u32x4{0u, 0u, 0u, 0u}}; }
    static __device__ __forceinline__ raw load_raw(const void *p, int64_t e)
    {
        return raw{__builtin_nontemporal_load(
            reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(p) + e))};
    }
    static __device__ __forceinline__ void fma8(const raw &r, float w, float (&acc)[VEC])
    {
        acc[0] = __builtin_fmaf(w, bf16_lo(r.v.x), acc[0]);
        acc[1] = __builtin_fmaf(w, bf16_hi(r.v.x), acc[1]);
        acc[2] = __builtin_fmaf(w, bf16_lo(r.v.y), acc[2]);
        acc[3] = __builtin_fmaf(w, bf16_hi(r.v.y), acc[3]);
        acc[4] = __builtin_fmaf(w, bf16_lo(r.v.z), acc[4]);
        acc[5] = __builtin_fmaf(w, bf16_hi(r.v.z), acc[5]);
        acc[6] = __builtin_fmaf(w, bf16_lo(r.v.w), acc[6]);
        acc[7] = __builtin_fmaf(w, bf16_hi(r.v.w), acc[7]);
    }
    static __device__ __forceinline__ void load8(const void *p, int64_t e, float (&v)[VEC])
    {
        const u32x4 *q = reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(p) + e);
        u32x4 w = __builtin_nontemporal_load(q);
        v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
        v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
        v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
        v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
    }
    static __device__ __forceinline__ void load4(const void *p, int64_t e, float (&v)[4])
    {
        const u32x2 w = __builtin_nontemporal_load(
            reinterpret_cast<const u32x2 *>(static_cast<const uint16_t *>(p) + e));
        v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
        v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    }
    // the 8 parameters as two quads at e0 and e1
    static __device__ __forceinline__ raw load_raw2(const void *p, int64_t e0, int64_t e1)
    {
        const uint16_t *h = static_cast<const uint16_t *>(p);
        const u32x2 a = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(h + e0));
        const u32x2 b = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(h + e1));
        return raw{u32x4{a.x, a.y, b.x, b.y}};
    }
    static __device__ __forceinline__ void load8_2(const void *p, int64_t e0, int64_t e1, float (&v)[VEC])
    {
        const raw r = load_raw2(p, e0, e1);
        v[0] = bf16_lo(r.v.x); v[1] = bf16_hi(r.v.x);
        v[2] = bf16_lo(r.v.y); v[3] = bf16_hi(r.v.y);
        v[4] = bf16_lo(r.v.z); v[5] = bf16_hi(r.v.z);
        v[6] = bf16_lo(r.v.w); v[7] = bf16_hi(r.v.w);
    }
    static __device__ __forceinline__ float load1(const void *p, int64_t e)
    {
        return bf16_lo(static_cast<const uint16_t *>(p)[e]);
    }
    static __device__ __forceinline__ void store8(void *p, int64_t e, const float (&v)[VEC])
    {
        u32x4 w;
        w.x = pack_bf16x2(v[0], v[1]);
        w.y = pack_bf16x2(v[2], v[3]);
        w.z = pack_bf16x2(v[4], v[5]);
        w.w = pack_bf16x2(v[6], v[7]);
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(p) + e));
    }
    static __device__ __forceinline__ void store1(void *p, int64_t e, float v)
    {
        static_cast<uint16_t *>(p)[e] = __builtin_bit_cast(uint16_t, (__bf16)v);
    }
};

__device__ __forceinline__ int64_t global_tid() { return (int64_t)blockIdx.x * blockDim.x + threadIdx.x; }
__device__ __forceinline__ int64_t grid_threads() { return (int64_t)gridDim.x * blockDim.x; }

// First parameters of the two 4-parameter quads that step v takes in a
// grid-stride loop of 256-lane workgroups over nvec steps of 8 fp32
// parameters.  In a full run of 256 steps these are quads l and l + 256 of
// the run (l = v mod 256), so the 16-byte accesses of a wave are contiguous
// and each of its store instructions writes 1 KiB of whole cache lines; in
// the last, short run they are quads 2l and 2l + 1.  With two 16-byte
// stores per lane 32 bytes apart instead, each store instruction of a wave
// leaves every line it touches half written; such stores were measured to
// move 11% more bytes to HBM than written (the read-modify-write of fp32
// sums), and to run 6-12% slower.
__device__ __forceinline__ void quad_pair(int64_t v, int64_t nvec, int64_t &e0, int64_t &e1)
{
    const int64_t run = v & ~(int64_t)255;
    const int64_t l = v & 255;
    const bool full = run + 256 <= nvec;
    e0 = run * VEC + (full ? l * 4 : l * 8);
    e1 = e0 + (full ? 1024 : 4);
}

// A raw buffer over the `bytes` bytes from p (clamped to 2^32 - 1): a load
// past its end reads zero without touching memory and a store past it is
// dropped, so accesses near the end of an array need no branch.  Loads
// through it carry the nt (non-temporal) bit, stores sc1 and nt: with K = 16
// bf16 clients at 2 workgroups per CU stores ran 10.85-10.87 ms with sc1 nt,
// 10.87-10.90 with sc1 or sc0 sc1, 10.93 with nt alone and 11.62 with no
// bits, on one allocation.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_rsrc(const void *p, int64_t bytes)
{
    const uint32_t n = bytes < 0xFFFFFFFFll ? (uint32_t)bytes : 0xFFFFFFFFu;
    // stride 0 (raw), the raw-buffer format word of gfx9 parts
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)n, 0x00020000);
}
constexpr int BUF_NT = 2;     // loads: nt
constexpr int BUF_STORE = 18; // stores: sc1 nt

// 8 parameters through a span: 8 consecutive ones at byte offset o, or two
// quads at byte offsets o0 and o1.
template <int DT> struct bio;
template <> struct bio<DT_F32> {
    static __device__ __forceinline__ f32x4 q(__amdgpu_buffer_rsrc_t r, int o)
    {
        return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, BUF_NT));
    }
    static __device__ __forceinline__ io<DT_F32>::raw load2(__amdgpu_buffer_rsrc_t r, int o0, int o1)
    {
        return io<DT_F32>::raw{q(r, o0), q(r, o1)};
    }
    static __device__ __forceinline__ io<DT_F32>::raw load(__amdgpu_buffer_rsrc_t r, int o)
    {
        return load2(r, o, o + 16);
    }
    static __device__ __forceinline__ void unpack(const io<DT_F32>::raw &w, float (&v)[VEC])
    {
        v[0] = w.a.x; v[1] = w.a.y; v[2] = w.a.z; v[3] = w.a.w;
        v[4] = w.b.x; v[5] = w.b.y; v[6] = w.b.z; v[7] = w.b.w;
    }
    static __device__ __forceinline__ void store2(__amdgpu_buffer_rsrc_t r, int o0, int o1, const float (&v)[VEC])
    {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{v[0], v[1], v[2], v[3]}), r, o0, 0, BUF_STORE);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{v[4], v[5], v[6], v[7]}), r, o1, 0, BUF_STORE);
    }
};
template <> struct bio<DT_BF16> {
    static __device__ __forceinline__ io<DT_BF16>::raw load(__amdgpu_buffer_rsrc_t r, int o)
    {
        return io<DT_BF16>::raw{__builtin_amdgcn_raw_buffer_load_b128(r, o, 0, BUF_NT)};
    }
    static __device__ __forceinline__ io<DT_BF16>::raw load2(__amdgpu_buffer_rsrc_t r, int o0, int o1)
    {
        const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(r, o0, 0, BUF_NT);
        const u32x2 b = __builtin_amdgcn_raw_buffer_load_b64(r, o1, 0, BUF_NT);
        return io<DT_BF16>::raw{u32x4{a.x, a.y, b.x, b.y}};
    }
    static __device__ __forceinline__ void unpack(const io<DT_BF16>::raw &w, float (&v)[VEC])
    {
        v[0] = bf16_lo(w.v.x); v[1] = bf16_hi(w.v.x);
        v[2] = bf16_lo(w.v.y); v[3] = bf16_hi(w.v.y);
        v[4] = bf16_lo(w.v.z); v[5] = bf16_hi(w.v.z);
        v[6] = bf16_lo(w.v.w); v[7] = bf16_hi(w.v.w);
    }
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, int o, const float (&v)[VEC])
    {
        const u32x4 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                         pack_bf16x2(v[6], v[7])};
        __builtin_amdgcn_raw_buffer_store_b128(w, r, o, 0, BUF_STORE);
    }
};

// ================================================================ resident dense

// One pass over K client buffers.  A workgroup takes 256 consecutive steps of
// 8 parameters (a grid-stride loop when the grid is capped); each lane owns 8
// parameters of its step (8 consecutive ones for a bf16 output, for an fp32
// one the two quads quad_pair describes, so that stores write whole lines),
// issues the loads of every client (KC of them when the client count is a
// compile-time constant KC > 0; batches of -KC clients for a client count
// known at run time) and of the base before its FMAs, then writes the 8
// results.  Every access goes through a buffer over the workgroup's part of
// its array, based at the workgroup's first parameter: the last workgroup's
// lanes past the end read zeros and drop their stores without a branch, and
// arrays of any length (beyond 2^32 bytes) stay within the 32-bit offsets.
// Buffer accesses ran 1% faster than global ones on the K = 16 bf16 2.0B
// workload (0.743 against 0.736 of HBM peak on one allocation).
template <int XDT, int ODT, int BDT, int MODE, int KC>
__global__ __launch_bounds__(256) void dense_vec_kernel(const DenseArgs a, int64_t nvec)
{
    constexpr bool SPLIT = ODT == DT_F32;
    constexpr int GB = KC < 0 ? -KC : 8;
    constexpr int XB = XDT == DT_F32 ? 4 : 2, BB = BDT == DT_F32 ? 4 : 2, OB = ODT == DT_F32 ? 4 : 2;
    const int K = KC > 0 ? KC : a.K;
    const int l = threadIdx.x;
    // the stride from gridDim.x and the fixed workgroup size: blockDim.x
    // would be a load from the dispatch packet that the first loads wait on
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t b = (int64_t)blockIdx.x * 256; b < nvec; b += stride) {
        const int64_t left = nvec - b; // steps from the workgroup's first on
        const int64_t e = b * VEC;     // its first parameter
        // the lane's two quads, as parameter offsets from e
        int p0 = l * 8, p1 = l * 8 + 4;
        if constexpr (SPLIT) {
            const bool full = left >= 256;
            p0 = full ? l * 4 : l * 8;
            p1 = p0 + (full ? 1024 : 4);
        }
        float acc[VEC];
#pragma unroll
        for (int j = 0; j < VEC; ++j)
            acc[j] = 0.0f;
        typename io<BDT>::raw braw;
        if constexpr (KC > 0) {
            typename io<XDT>::raw xr[KC];
#pragma unroll
            for (int k = 0; k < KC; ++k) {
                const auto r = span_rsrc(static_cast<const char *>(a.x[k]) + e * XB, left * VEC * XB);
                xr[k] = SPLIT ? bio<XDT>::load2(r, p0 * XB, p1 * XB) : bio<XDT>::load(r, p0 * XB);
            }
            if constexpr (MODE == MODE_DELTAS) {
                const auto r = span_rsrc(static_cast<const char *>(a.base) + e * BB, left * VEC * BB);
                braw = SPLIT ? bio<BDT>::load2(r, p0 * BB, p1 * BB) : bio<BDT>::load(r, p0 * BB);
            }
            // every load is issued before the first FMA waits on one
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < KC; ++k)
                io<XDT>::fma8(xr[k], a.w[k], acc);
        } else {
            if constexpr (MODE == MODE_DELTAS) {
                const auto r = span_rsrc(static_cast<const char *>(a.base) + e * BB, left * VEC * BB);
                braw = SPLIT ? bio<BDT>::load2(r, p0 * BB, p1 * BB) : bio<BDT>::load(r, p0 * BB);
            }
            for (int k0 = 0; k0 < K; k0 += GB) {
                typename io<XDT>::raw xr[GB];
                // the batch's client pointers in one go (wide scalar loads)
                struct Batch {
                    const void *p[GB];
                };
                const Batch xb = *reinterpret_cast<const Batch *>(&a.x[k0]);
                // the last batch's slots past K load zeros through an empty
                // buffer and add them with weight -0 (the host fills w[k] =
                // -0 for k >= K), which leaves every accumulator bit as it
                // is: -0 * 0 + acc is acc, -0 included
#pragma unroll
                for (int k = 0; k < GB; ++k) {
                    const bool in = k0 + k < K;
                    const auto r = span_rsrc(static_cast<const char *>(xb.p[in ? k : 0]) + e * XB,
                                             in ? left * VEC * XB : 0);
                    xr[k] = SPLIT ? bio<XDT>::load2(r, p0 * XB, p1 * XB) : bio<XDT>::load(r, p0 * XB);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int k = 0; k < GB; ++k)
                    io<XDT>::fma8(xr[k], a.w[k0 + k], acc);
            }
        }
        float r[VEC];
        if constexpr (MODE == MODE_DELTAS) {
            float bv[VEC];
            bio<BDT>::unpack(braw, bv);
#pragma unroll
            for (int j = 0; j < VEC; ++j)
                r[j] = bv[j] + acc[j] / a.S;
        } else {
#pragma unroll
            for (int j = 0; j < VEC; ++j)
                r[j] = acc[j] / a.S;
        }
        const auto ro = span_rsrc(static_cast<char *>(a.out) + e * OB, left * VEC * OB);
        if constexpr (SPLIT)
            bio<DT_F32>::store2(ro, p0 * 4, p1 * 4, r);
        else
            bio<DT_BF16>::store(ro, p0 * 2, r);
    }
}

// Element-wise form (unaligned buffers and the last N % 8 parameters), same
// operation order as the vector form, so results are bit-identical.
template <int XDT, int ODT, int BDT, int MODE>
__global__ __launch_bounds__(256) void dense_scalar_kernel(const DenseArgs a, int64_t first,
                                                           int64_t count)
{
    for (int64_t t = global_tid(); t < count; t += grid_threads()) {
        const int64_t e = first + t;
        float acc = 0.0f;
        for (int k = 0; k < a.K; ++k)
            acc = __builtin_fmaf(a.w[k], io<XDT>::load1(a.x[k], e), acc);
        float r = acc / a.S;
        if constexpr (MODE == MODE_DELTAS)
            r = io<BDT>::load1(a.base, e) + r;
        io<ODT>::store1(a.out, e, r);
    }
}

// ================================================================ per-segment masks

constexpr int SEG_WIN = 64; // segments staged in LDS at a time (windowed kernel)

// Last segment index t in [0, T-1] with bounds[t] <= e (a thread alone).
__device__ __forceinline__ int64_t thread_find_segment(const int64_t *bounds, int64_t T, int64_t e)
{
    int64_t lo = 0, hi = T - 1;
    while (lo < hi) {
        int64_t mid = lo + (hi - lo + 1) / 2;
        if (bounds[mid] <= e)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// Same search done by one whole wavefront: each round the 64 lanes probe 64
// evenly spaced bounds and a ballot narrows the range 64-fold, so a table of
// T segments costs ceil(log64(T+1)) dependent loads instead of log2(T).
__device__ int64_t wave_find_segment(const int64_t *bounds, int64_t T, int64_t e, int lane)
{
    int64_t lo = 0, hi = T; // answer in [lo, hi)
    while (hi - lo > 1) {
        const int64_t span = hi - lo;
        const int64_t step = (span + 63) / 64;
        const int64_t pos = lo + (int64_t)lane * step;
        const bool le = pos < hi && bounds[pos] <= e;
        int c = __popcll(__ballot(le));
        if (c < 1)
            c = 1; // malformed table: stay in range
        const int64_t nlo = lo + (int64_t)(c - 1) * step;
        const int64_t nhi = lo + (int64_t)c * step;
        lo = nlo;
        hi = nhi < hi ? nhi : hi;
    }
    return lo;
}

// The clients' presence bytes of segment t are read 8 at a time, each
// batch issued before any is tested: read one after another, with a test
// between, every load waited for the one before it, and a workgroup's table
// took K round trips before its first client load.
__device__ __forceinline__ void segment_weights(const MaskedArgs &a, int64_t t, uint64_t &mask,
                                                uint32_t &W)
{
    uint64_t m = 0;
    uint32_t s = 0;
    for (int k0 = 0; k0 < a.K; k0 += 8) {
        uint32_t p[8];
        // unconditional loads (a client index past K reads the last
        // client's byte and drops it): a load under a branch is waited for
        // before the next one is issued
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int k = min(k0 + j, a.K - 1);
            const uint32_t byte = a.present[(int64_t)a.row[k] * a.T + t];
            p[j] = k0 + j < a.K ? byte : 0u;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (p[j]) {
                m |= 1ull << (k0 + j);
                s += a.wi[k0 + j];
            }
        }
    }
    mask = m;
    W = s;
}

template <int XDT, int ODT, int BDT, int MODE>
__device__ __forceinline__ void masked_element(const MaskedArgs &a, int64_t e)
{
    uint64_t mask;
    uint32_t W;
    segment_weights(a, thread_find_segment(a.bounds, a.T, e), mask, W);
    float r;
    if (W > 0) {
        float acc = 0.0f;
        for (int k = 0; k < a.K; ++k)
            if ((mask >> k) & 1)
                acc = __builtin_fmaf(a.w[k], io<XDT>::load1(a.x[k], e), acc);
        r = acc / (a.zero_fill ? a.S_all : (float)W);
        if constexpr (MODE == MODE_DELTAS)
            r = io<BDT>::load1(a.base, e) + r;
    } else {
        r = io<BDT>::load1(a.base, e);
    }
    io<ODT>::store1(a.out, e, r);
}

// Element-wise path for a vector (the quads at e0 and e1) whose 8 parameters
// do not all lie in one segment (or run past the end of the buffer).
template <int XDT, int ODT, int BDT, int MODE>
__device__ __forceinline__ void masked_vector_elementwise(const MaskedArgs &a, int64_t e0, int64_t e1)
{
    for (int j = 0; j < 4; ++j)
        if (e0 + j < a.N)
            masked_element<XDT, ODT, BDT, MODE>(a, e0 + j);
    for (int j = 0; j < 4; ++j)
        if (e1 + j < a.N)
            masked_element<XDT, ODT, BDT, MODE>(a, e1 + j);
}

// Each workgroup owns a contiguous run of `vpb` 8-parameter vectors, walked
// as spans of blockDim vectors (one per lane).  Wave 0 locates the segment
// holding the run's first parameter; the block stages up to SEG_WIN
// consecutive segments (bounds, client mask, weight sum) in LDS and walks its
// spans through them, window after window.  A span inside one segment -- the
// usual case, segments being whole tensors -- has one client mask for all
// lanes, held in scalar registers: the lanes read only the clients present
// there, with no divergence.  A span that straddles a segment boundary falls
// back to per-element lookups.
template <int XDT, int ODT, int BDT, int MODE>
__global__ __launch_bounds__(256) void masked_vec_kernel(const MaskedArgs a)
{
    constexpr bool SPLIT = ODT == DT_F32;
    __shared__ int64_t s_lo[SEG_WIN + 1];
    __shared__ uint64_t s_mask[SEG_WIN];
    __shared__ uint32_t s_W[SEG_WIN];
    __shared__ int64_t s_t0;

    const int tid = threadIdx.x;
    const int64_t nvec_all = (a.N + VEC - 1) / VEC;
    const int64_t v_begin = (int64_t)blockIdx.x * a.vpb;
    if (v_begin >= nvec_all)
        return;
    const int64_t v_end = min(v_begin + a.vpb, nvec_all);
    const int64_t e_end = min(v_end * VEC, a.N);
    int64_t e_cur = v_begin * VEC;
    int64_t t_next = -1;

    while (e_cur < e_end) {
        if (tid < 64) {
            const int64_t t0 = t_next >= 0 ? t_next : wave_find_segment(a.bounds, a.T, e_cur, tid);
            if (tid == 0)
                s_t0 = t0;
        }
        __syncthreads();
        const int64_t t0 = s_t0;
        const int cnt = (int)min((int64_t)SEG_WIN, (int64_t)a.T - t0);
        if (tid <= cnt)
            s_lo[tid] = a.bounds[t0 + tid];
        if (tid < cnt)
            segment_weights(a, t0 + tid, s_mask[tid], s_W[tid]);
        __syncthreads();

        int64_t win_end = min(s_lo[cnt], e_end);
        if (win_end <= e_cur)
            win_end = e_end; // malformed table: finish with element-wise lookups
        const int64_t vw0 = (e_cur + VEC - 1) / VEC;
        const int64_t vw1 = min((win_end + VEC - 1) / VEC, v_end);

        for (int64_t s0 = vw0; s0 < vw1; s0 += blockDim.x) {
            // block-uniform span [s0, s1) of vectors and its parameters
            const int64_t s1 = min(s0 + (int64_t)blockDim.x, vw1);
            const int64_t E0 = s0 * VEC;
            const int64_t E1 = min(s1 * VEC, a.N);
            int lo = 0, hi = cnt - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) / 2;
                if (s_lo[mid] <= E0)
                    lo = mid;
                else
                    hi = mid - 1;
            }
            const bool one_segment = s_lo[lo] <= E0 && E1 <= s_lo[lo + 1];
            const int64_t v = s0 + tid;
            if (v >= s1)
                continue;
            // an fp32 output: in a full span of 256 vectors the lane takes
            // the quads tid and 256 + tid of the span (whole-line stores)
            int64_t e0 = v * VEC, e1 = e0 + 4;
            if (SPLIT && s1 - s0 == 256) {
                e0 = s0 * VEC + tid * 4;
                e1 = e0 + 1024;
            }
            if (one_segment && e1 + 4 <= a.N) {
                const uint64_t smask = s_mask[lo];
                const uint32_t mlo = __builtin_amdgcn_readfirstlane((uint32_t)smask);
                const uint32_t mhi = __builtin_amdgcn_readfirstlane((uint32_t)(smask >> 32));
                const uint64_t mask = ((uint64_t)mhi << 32) | mlo;
                const uint32_t W = __builtin_amdgcn_readfirstlane(s_W[lo]);
                float r[VEC];
                if (W > 0) {
                    float acc[VEC];
#pragma unroll
                    for (int j = 0; j < VEC; ++j)
                        acc[j] = 0.0f;
                    for (int k0 = 0; k0 < a.K; k0 += 8) {
                        // as in masked_table_kernel: absent clients are not
                        // read, their FMA runs as 0 * 0 so the loads issue together
                        typename io<XDT>::raw xr[8];
                        float wk[8];
#pragma unroll
                        for (int k = 0; k < 8; ++k) {
                            const bool on = k0 + k < a.K && ((mask >> (k0 + k)) & 1);
                            xr[k] = io<XDT>::zero_raw();
                            wk[k] = on ? a.w[k0 + k] : 0.0f;
                            if (on)
                                xr[k] = SPLIT ? io<XDT>::load_raw2(a.x[k0 + k], e0, e1)
                                              : io<XDT>::load_raw(a.x[k0 + k], e0);
                        }
#pragma unroll
                        for (int k = 0; k < 8; ++k)
                            io<XDT>::fma8(xr[k], wk[k], acc);
                    }
                    const float Wf = a.zero_fill ? a.S_all : (float)W;
                    if constexpr (MODE == MODE_DELTAS) {
                        float b[VEC];
                        if constexpr (SPLIT)
                            io<BDT>::load8_2(a.base, e0, e1, b);
                        else
                            io<BDT>::load8(a.base, e0, b);
#pragma unroll
                        for (int j = 0; j < VEC; ++j)
                            r[j] = b[j] + acc[j] / Wf;
                    } else {
#pragma unroll
                        for (int j = 0; j < VEC; ++j)
                            r[j] = acc[j] / Wf;
                    }
                } else if constexpr (SPLIT) {
                    io<BDT>::load8_2(a.base, e0, e1, r);
                } else {
                    io<BDT>::load8(a.base, e0, r);
                }
                if constexpr (SPLIT)
                    io<ODT>::store8_2(a.out, e0, e1, r);
                else
                    io<ODT>::store8(a.out, e0, r);
            } else {
                masked_vector_elementwise<XDT, ODT, BDT, MODE>(a, e0, e1);
            }
        }
        e_cur = win_end;
        t_next = t0 + cnt;
        if (t_next >= a.T)
            t_next = a.T - 1;
        __syncthreads(); // LDS window is rewritten next
    }
}

// Last segment index t in [lo, T-1] with s_lo[t] <= e, over a table staged
// in LDS (lo <= T-1).
__device__ __forceinline__ int lds_find_segment(const int64_t *s_lo, int lo, int T, int64_t e)
{
    int hi = T - 1;
    while (lo < hi) {
        const int mid = lo + (hi - lo + 1) / 2;
        if (s_lo[mid] <= e)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// One parameter of the masked aggregate, its segment looked up in the LDS
// table.
template <int XDT, int ODT, int BDT, int MODE>
__device__ __forceinline__ void masked_element_lds(const MaskedArgs &a, const int64_t *s_lo,
                                                   const uint64_t *s_mask, const uint32_t *s_W,
                                                   int64_t e)
{
    const int t = lds_find_segment(s_lo, 0, (int)a.T, e);
    const uint64_t m = s_mask[t];
    const uint32_t W = s_W[t];
    float r;
    if (W > 0) {
        float acc = 0.0f;
        for (int k = 0; k < a.K; ++k)
            if ((m >> k) & 1)
                acc = __builtin_fmaf(a.w[k], io<XDT>::load1(a.x[k], e), acc);
        r = acc / (a.zero_fill ? a.S_all : (float)W);
        if constexpr (MODE == MODE_DELTAS)
            r = io<BDT>::load1(a.base, e) + r;
    } else {
        r = io<BDT>::load1(a.base, e);
    }
    io<ODT>::store1(a.out, e, r);
}

// Tables of at most TAB_SEGS segments (LoRA-style adapter sets: a few hundred
// tensors) are staged whole in LDS by every workgroup, in one round of
// independent loads -- bounds and client presence together -- instead of a
// search followed by a windowed fetch.  Each thread then walks its vectors
// (the grid strides over all of them) NV at a time with a segment cursor that
// only moves forward, so a vector costs one LDS compare in the usual case.
// The loads of all NV vectors are issued before the first FMA: absent
// clients are skipped, which leaves a wave fewer bytes in flight than the
// dense kernel has, and NV restores them.  Lanes whose vector straddles a
// segment boundary or the buffer end go element by element.
template <int XDT, int ODT, int BDT, int MODE, int NV>
__global__ __launch_bounds__(256) void masked_table_kernel(const MaskedArgs a)
{
    __shared__ int64_t s_lo[TAB_SEGS + 1];
    __shared__ uint64_t s_mask[TAB_SEGS];
    __shared__ uint32_t s_W[TAB_SEGS];

    const int tid = threadIdx.x;
    const int T = (int)a.T;
    // a segment's bound and its clients' presence bytes in one round trip
    for (int t = tid; t <= T; t += blockDim.x) {
        const int64_t lo = a.bounds[t];
        if (t < T)
            segment_weights(a, t, s_mask[t], s_W[t]);
        s_lo[t] = lo;
    }
    __syncthreads();

    // Grid-stride over the vectors (the grid holds about N / (8 vpb)
    // workgroups): the resident workgroups sweep one window of the buffers
    // together, which the DRAM serves better than as many separate runs.
    const int64_t nvec_all = (a.N + VEC - 1) / VEC;
    const int64_t v_end = nvec_all;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    // an fp32 output: a lane takes the quads quad_pair gives (whole-line
    // stores); the first quad moves the segment cursor, and a vector is fast
    // when both quads lie in its segment
    constexpr bool SPLIT = ODT == DT_F32;
    int t = -1;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + tid; v < v_end; v += NV * stride) {
        int64_t ev[NV], ew[NV];
        bool has[NV], fast[NV];
        uint64_t m[NV];
        uint32_t W[NV];
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            ev[u] = (v + u * stride) * VEC;
            ew[u] = ev[u] + 4;
            if constexpr (SPLIT)
                quad_pair(v + u * stride, v_end, ev[u], ew[u]);
            has[u] = v + u * stride < v_end;
            fast[u] = false;
            m[u] = 0;
            W[u] = 0;
            if (has[u]) {
                if (t < 0 || s_lo[t + 1] <= ev[u])
                    t = lds_find_segment(s_lo, min(t + 1, T - 1), T, ev[u]);
                fast[u] = s_lo[t] <= ev[u] && ew[u] + 4 <= s_lo[t + 1] && ew[u] + 4 <= a.N;
                if (fast[u]) {
                    m[u] = s_mask[t];
                    W[u] = s_W[t];
                }
            }
        }
        float acc[NV][VEC];
#pragma unroll
        for (int u = 0; u < NV; ++u)
#pragma unroll
            for (int j = 0; j < VEC; ++j)
                acc[u][j] = 0.0f;
        for (int k0 = 0; k0 < a.K; k0 += 8) {
            // Only present clients are read.  Every FMA runs, an absent
            // client's as 0 * 0 (exact: acc starts at +0 and cannot become
            // -0), so each load is consumed on every path and the compiler
            // does not serialize the next loads behind a wait for all of them.
            typename io<XDT>::raw xr[NV][8];
            float wk[NV][8];
#pragma unroll
            for (int u = 0; u < NV; ++u)
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const bool on = k0 + k < a.K && ((m[u] >> (k0 + k)) & 1);
                    xr[u][k] = io<XDT>::zero_raw();
                    wk[u][k] = on ? a.w[k0 + k] : 0.0f;
                    if (on)
                        xr[u][k] = SPLIT ? io<XDT>::load_raw2(a.x[k0 + k], ev[u], ew[u])
                                         : io<XDT>::load_raw(a.x[k0 + k], ev[u]);
                }
#pragma unroll
            for (int u = 0; u < NV; ++u)
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    io<XDT>::fma8(xr[u][k], wk[u][k], acc[u]);
        }
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            if (!has[u])
                continue;
            if (!fast[u]) {
                for (int j = 0; j < 4 && ev[u] + j < a.N; ++j)
                    masked_element_lds<XDT, ODT, BDT, MODE>(a, s_lo, s_mask, s_W, ev[u] + j);
                for (int j = 0; j < 4 && ew[u] + j < a.N; ++j)
                    masked_element_lds<XDT, ODT, BDT, MODE>(a, s_lo, s_mask, s_W, ew[u] + j);
                continue;
            }
            float r[VEC];
            if (W[u] > 0) {
                const float Wf = a.zero_fill ? a.S_all : (float)W[u];
                if constexpr (MODE == MODE_DELTAS) {
                    float b[VEC];
                    if constexpr (SPLIT)
                        io<BDT>::load8_2(a.base, ev[u], ew[u], b);
                    else
                        io<BDT>::load8(a.base, ev[u], b);
#pragma unroll
                    for (int j = 0; j < VEC; ++j)
                        r[j] = b[j] + acc[u][j] / Wf;
                } else {
#pragma unroll
                    for (int j = 0; j < VEC; ++j)
                        r[j] = acc[u][j] / Wf;
                }
            } else if constexpr (SPLIT) {
                io<BDT>::load8_2(a.base, ev[u], ew[u], r);
            } else {
                io<BDT>::load8(a.base, ev[u], r);
            }
            if constexpr (SPLIT)
                io<ODT>::store8_2(a.out, ev[u], ew[u], r);
            else
                io<ODT>::store8(a.out, ev[u], r);
        }
    }
}

template <int XDT, int ODT, int BDT, int MODE>
__global__ __launch_bounds__(256) void masked_scalar_kernel(const MaskedArgs a)
{
    for (int64_t e = global_tid(); e < a.N; e += grid_threads())
        masked_element<XDT, ODT, BDT, MODE>(a, e);
}

// ================================================================ streaming

// acc[offset + e] += n_k * chunk[e] over one chunk; in partial modes also the
// per-parameter weight sum and client count of the parameters sent.
template <int DT, int PART>
__global__ __launch_bounds__(256) void stream_acc_vec_kernel(const StreamArgs a, int64_t nvec)
{
    // a workgroup takes 256 consecutive steps of 8 parameters through
    // buffers based at its first parameter; a lane's two quads are
    // quad_pair's (whole-line stores of the sums)
    constexpr int XB = DT == DT_F32 ? 4 : 2;
    const int l = threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t b = (int64_t)blockIdx.x * 256; b < nvec; b += stride) {
        const int64_t left = nvec - b, e = b * VEC;
        const bool full = left >= 256;
        const int pq[2] = {full ? l * 4 : l * 8, (full ? l * 4 : l * 8) + (full ? 1024 : 4)};
        const auto rx = span_rsrc(static_cast<const char *>(a.chunk) + e * XB, left * VEC * XB);
        const auto ra = span_rsrc(a.acc + a.offset + e, left * VEC * 4);
        float xv[2][4];
        f32x4 acc[2];
        uint32_t sent[2] = {0xfu, 0xfu};
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            if constexpr (DT == DT_F32) {
                const f32x4 x = bio<DT_F32>::q(rx, pq[q] * 4);
                xv[q][0] = x.x; xv[q][1] = x.y; xv[q][2] = x.z; xv[q][3] = x.w;
            } else {
                const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rx, pq[q] * 2, 0, BUF_NT);
                xv[q][0] = bf16_lo(x.x); xv[q][1] = bf16_hi(x.x);
                xv[q][2] = bf16_lo(x.y); xv[q][3] = bf16_hi(x.y);
            }
            acc[q] = bio<DT_F32>::q(ra, pq[q] * 4);
            if constexpr (PART == PART_MASK) {
                const auto rm = span_rsrc(a.mask + e, left * VEC);
                const uint32_t mb = __builtin_amdgcn_raw_buffer_load_b32(rm, pq[q], 0, 0);
                sent[q] = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    sent[q] |= (((mb >> (8 * j)) & 0xffu) != 0) << j;
            }
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            f32x4 &sm = acc[q];
            if (sent[q] & 1) sm.x = __builtin_fmaf(a.w, xv[q][0], sm.x);
            if (sent[q] & 2) sm.y = __builtin_fmaf(a.w, xv[q][1], sm.y);
            if (sent[q] & 4) sm.z = __builtin_fmaf(a.w, xv[q][2], sm.z);
            if (sent[q] & 8) sm.w = __builtin_fmaf(a.w, xv[q][3], sm.w);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, sm), ra, pq[q] * 4, 0, BUF_STORE);
        }
        if constexpr (PART != PART_DENSE) {
            const auto rw = span_rsrc(a.wsum + a.offset + e, left * VEC * 4);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rw, pq[q] * 4, 0, 0);
                w.x += (sent[q] & 1) ? a.wi : 0u;
                w.y += (sent[q] & 2) ? a.wi : 0u;
                w.z += (sent[q] & 4) ? a.wi : 0u;
                w.w += (sent[q] & 8) ? a.wi : 0u;
                __builtin_amdgcn_raw_buffer_store_b128(w, rw, pq[q] * 4, 0, 0);
                if (a.count) {
                    // one byte per parameter; a client adds at most 1 and
                    // there are at most 255 clients, so no byte carries into
                    // the next
                    const auto rc = span_rsrc(a.count + a.offset + e, left * VEC);
                    uint32_t add = 0;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        add |= ((sent[q] >> j) & 1u) << (8 * j);
                    const uint32_t c = __builtin_amdgcn_raw_buffer_load_b32(rc, pq[q], 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b32(c + add, rc, pq[q], 0, 0);
                }
            }
        }
    }
}

template <int DT, int PART>
__global__ __launch_bounds__(256) void stream_acc_scalar_kernel(const StreamArgs a, int64_t first,
                                                                int64_t count)
{
    for (int64_t t = global_tid(); t < count; t += grid_threads()) {
        const int64_t e = first + t;
        const int64_t g = a.offset + e;
        if constexpr (PART == PART_MASK) {
            if (!a.mask[e])
                continue;
        }
        a.acc[g] = __builtin_fmaf(a.w, io<DT>::load1(a.chunk, e), a.acc[g]);
        if constexpr (PART != PART_DENSE) {
            a.wsum[g] += a.wi;
            if (a.count)
                a.count[g] += 1;
        }
    }
}

// Client-at-a-time sparse accumulate: value j goes to parameter
// offset + idx[j].  Indices are unique within a call, so no two lanes touch
// the same parameter and no atomics are needed; bad entries are skipped and
// flagged.
template <int DT>
__global__ __launch_bounds__(256) void stream_acc_index_kernel(const StreamArgs a)
{
    // an index is good when it lies in [0, N - offset) and above its
    // predecessor; the bounds are tested on the index itself, so neither a
    // negative one (also in a run that increases) nor offset + index
    // wrapping past 2^63 can address memory outside the accumulator
    if (a.gate && *a.gate == 0)
        return; // the tiled path took this list
    const int64_t span = a.N - a.offset;
    for (int64_t j = global_tid(); j < a.len; j += grid_threads()) {
        const int64_t ix = a.idx[j];
        const int64_t prev = j > 0 ? a.idx[j - 1] : -1;
        if (ix < 0 || ix >= span || ix <= prev) {
            *a.err = FA_ERR_INDEX;
            continue;
        }
        const int64_t g = a.offset + ix;
        a.acc[g] = __builtin_fmaf(a.w, io<DT>::load1(a.chunk, j), a.acc[g]);
        a.wsum[g] += a.wi;
        if (a.count)
            a.count[g] += 1;
    }
}

// Two-level aggregation: a lower-level accumulator's unnormalised partial
// sums enter this one as a single pseudo-client, acc += src (one fp32
// addition per parameter), and in partial mode its weight sums and client
// counts add to these.  The counts add as packed bytes: the handle keeps the
// total number of clients at most 255, so no byte carries into the next.
template <int PARTIAL>
__global__ __launch_bounds__(256) void stream_merge_vec_kernel(const StreamArgs a, int64_t nvec)
{
    // a workgroup takes 256 consecutive steps of 8 parameters through
    // buffers based at its first parameter (as the dense kernel does); a
    // lane's two quads are quad_pair's (whole-line stores)
    const float *src = static_cast<const float *>(a.chunk);
    const int l = threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t b = (int64_t)blockIdx.x * 256; b < nvec; b += stride) {
        const int64_t left = nvec - b, e = b * VEC;
        const bool full = left >= 256;
        const int p0 = full ? l * 4 : l * 8, p1 = p0 + (full ? 1024 : 4);
        const auto rs = span_rsrc(src + e, left * VEC * 4);
        const auto ra = span_rsrc(a.acc + a.offset + e, left * VEC * 4);
        const f32x4 s0 = bio<DT_F32>::q(rs, p0 * 4), s1 = bio<DT_F32>::q(rs, p1 * 4);
        f32x4 lo = bio<DT_F32>::q(ra, p0 * 4), hi = bio<DT_F32>::q(ra, p1 * 4);
        lo = f32x4{lo.x + s0.x, lo.y + s0.y, lo.z + s0.z, lo.w + s0.w};
        hi = f32x4{hi.x + s1.x, hi.y + s1.y, hi.z + s1.z, hi.w + s1.w};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, lo), ra, p0 * 4, 0, BUF_STORE);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, hi), ra, p1 * 4, 0, BUF_STORE);
        if constexpr (PARTIAL) {
            const auto rsw = span_rsrc(a.src_wsum + e, left * VEC * 4);
            const auto rw = span_rsrc(a.wsum + a.offset + e, left * VEC * 4);
            const u32x4 a0 = __builtin_amdgcn_raw_buffer_load_b128(rsw, p0 * 4, 0, BUF_NT);
            const u32x4 a1 = __builtin_amdgcn_raw_buffer_load_b128(rsw, p1 * 4, 0, BUF_NT);
            u32x4 w0 = __builtin_amdgcn_raw_buffer_load_b128(rw, p0 * 4, 0, 0);
            u32x4 w1 = __builtin_amdgcn_raw_buffer_load_b128(rw, p1 * 4, 0, 0);
            w0 = u32x4{w0.x + a0.x, w0.y + a0.y, w0.z + a0.z, w0.w + a0.w};
            w1 = u32x4{w1.x + a1.x, w1.y + a1.y, w1.z + a1.z, w1.w + a1.w};
            __builtin_amdgcn_raw_buffer_store_b128(w0, rw, p0 * 4, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b128(w1, rw, p1 * 4, 0, 0);
            if (a.count) {
                const auto rsc = span_rsrc(a.src_count + e, left * VEC);
                const auto rc = span_rsrc(a.count + a.offset + e, left * VEC);
                const uint32_t c0 = __builtin_amdgcn_raw_buffer_load_b32(rsc, p0, 0, 0);
                const uint32_t c1 = __builtin_amdgcn_raw_buffer_load_b32(rsc, p1, 0, 0);
                const uint32_t d0 = __builtin_amdgcn_raw_buffer_load_b32(rc, p0, 0, 0);
                const uint32_t d1 = __builtin_amdgcn_raw_buffer_load_b32(rc, p1, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(d0 + c0, rc, p0, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(d1 + c1, rc, p1, 0, 0);
            }
        }
    }
}

template <int PARTIAL>
__global__ __launch_bounds__(256) void stream_merge_scalar_kernel(const StreamArgs a, int64_t first,
                                                                  int64_t count)
{
    const float *src = static_cast<const float *>(a.chunk);
    for (int64_t t = global_tid(); t < count; t += grid_threads()) {
        const int64_t e = first + t;
        const int64_t g = a.offset + e;
        a.acc[g] = a.acc[g] + src[e];
        if constexpr (PARTIAL) {
            a.wsum[g] += a.src_wsum[e];
            if (a.count)
                a.count[g] = (uint8_t)(a.count[g] + a.src_count[e]);
        }
    }
}

template <int BDT, int ODT, int MODE, int PARTIAL>
__device__ __forceinline__ float finalize_one(float acc, uint32_t W, float S, float b, int zero_fill)
{
    if constexpr (PARTIAL) {
        if (W == 0)
            return b;
        const float q = acc / (zero_fill ? S : (float)W);
        return MODE == MODE_DELTAS ? b + q : q;
    } else {
        const float q = acc / S;
        return MODE == MODE_DELTAS ? b + q : q;
    }
}

template <int BDT, int ODT, int MODE, int PARTIAL>
__global__ __launch_bounds__(256) void stream_finalize_vec_kernel(const FinalizeArgs a, int64_t nvec)
{
    // a workgroup takes 256 consecutive steps of 8 parameters through
    // buffers based at its first parameter; an fp32 output is written as
    // quad_pair's two quads per lane (whole-line stores), a bf16 output's 8
    // values as one contiguous 16-byte store
    constexpr bool SPLIT = ODT == DT_F32;
    constexpr int BB = BDT == DT_F32 ? 4 : 2, OB = ODT == DT_F32 ? 4 : 2;
    const int l = threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t b = (int64_t)blockIdx.x * 256; b < nvec; b += stride) {
        const int64_t left = nvec - b, e = b * VEC;
        int p0 = l * 8, p1 = l * 8 + 4;
        if constexpr (SPLIT) {
            const bool full = left >= 256;
            p0 = full ? l * 4 : l * 8;
            p1 = p0 + (full ? 1024 : 4);
        }
        const auto ra = span_rsrc(a.acc + e, left * VEC * 4);
        const f32x4 lo = bio<DT_F32>::q(ra, p0 * 4);
        const f32x4 hi = bio<DT_F32>::q(ra, p1 * 4);
        const float acc[VEC] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        uint32_t W[VEC] = {0, 0, 0, 0, 0, 0, 0, 0};
        if constexpr (PARTIAL) {
            const auto rw = span_rsrc(a.wsum + e, left * VEC * 4);
            const u32x4 w0 = __builtin_amdgcn_raw_buffer_load_b128(rw, p0 * 4, 0, 0);
            const u32x4 w1 = __builtin_amdgcn_raw_buffer_load_b128(rw, p1 * 4, 0, 0);
            W[0] = w0.x; W[1] = w0.y; W[2] = w0.z; W[3] = w0.w;
            W[4] = w1.x; W[5] = w1.y; W[6] = w1.z; W[7] = w1.w;
        }
        float bv[VEC] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (MODE == MODE_DELTAS || PARTIAL) {
            const auto rb = span_rsrc(static_cast<const char *>(a.base) + e * BB, left * VEC * BB);
            bio<BDT>::unpack(SPLIT ? bio<BDT>::load2(rb, p0 * BB, p1 * BB) : bio<BDT>::load(rb, p0 * BB), bv);
        }
        float r[VEC];
#pragma unroll
        for (int j = 0; j < VEC; ++j)
            r[j] = finalize_one<BDT, ODT, MODE, PARTIAL>(acc[j], W[j], a.S, bv[j], a.zero_fill);
        const auto ro = span_rsrc(static_cast<char *>(a.out) + e * OB, left * VEC * OB);
        if constexpr (SPLIT)
            bio<DT_F32>::store2(ro, p0 * 4, p1 * 4, r);
        else
            bio<DT_BF16>::store(ro, p0 * 2, r);
    }
}

template <int BDT, int ODT, int MODE, int PARTIAL>
__global__ __launch_bounds__(256) void stream_finalize_scalar_kernel(const FinalizeArgs a,
                                                                     int64_t first, int64_t count)
{
    for (int64_t t = global_tid(); t < count; t += grid_threads()) {
        const int64_t e = first + t;
        const uint32_t W = PARTIAL ? a.wsum[e] : 0u;
        const float b = (MODE == MODE_DELTAS || PARTIAL) ? io<BDT>::load1(a.base, e) : 0.0f;
        io<ODT>::store1(a.out, e, finalize_one<BDT, ODT, MODE, PARTIAL>(a.acc[e], W, a.S, b, a.zero_fill));
    }
}

// ================================================================ sparse merge

// First position in ix[lo, hi) whose index is >= target (hi when there is
// none), for a list sorted ascending whose values in [lo, hi) lie above vlo
// and at most vhi (a whole list over [0, N): lo = 0, hi = n, vlo = -1,
// vhi = N).  Every probe lies inside the bracket that holds the answer, so
// the choice of probe changes only how fast it is found: the first
// SPARSE_INTERP_STEPS probes interpolate between the index values known at
// the bracket's ends (top-k supports are close to uniform, so a few probes
// land next to the answer), the rest bisect, which bounds the probes for any
// list.  An unsorted list gives some position in [lo, hi]; the merge reports
// such lists whatever the offsets are.
constexpr int SPARSE_INTERP_STEPS = 6;

__device__ __forceinline__ int64_t sparse_lower_bound(const int64_t *ix, int64_t lo, int64_t hi,
                                                      int64_t target, int64_t vlo, int64_t vhi)
{
    for (int step = 0; lo < hi; ++step) {
        int64_t mid = lo + (hi - lo) / 2;
        if (step < SPARSE_INTERP_STEPS && vhi > vlo && target > vlo && target <= vhi) {
            const double f = (double)(target - vlo) / (double)(vhi - vlo);
            const int64_t m = lo + (int64_t)(f * (double)(hi - lo));
            mid = m < lo ? lo : (m > hi - 1 ? hi - 1 : m);
        }
        const int64_t v = ix[mid];
        if (v < target) {
            lo = mid + 1;
            vlo = v;
        } else {
            hi = mid;
            vhi = v;
        }
    }
    return lo;
}

// For every client k and range boundary b (0..NB), the first position of k's
// sorted index list at or after parameter b*R.  Also flags lists that hold
// negative indices or indices >= N (those fall outside every range).
//
// A wave takes 64 consecutive boundaries of one client: its first and last
// lanes search the whole list for the outer two, and the other lanes search
// only between those two answers, where every index lies in [first target,
// last target).  The inner searches start within a few hundred positions of
// their answers, so a wave costs about half the random line reads of 64
// independent whole-list searches (the kernel is bound by those reads).
__global__ __launch_bounds__(256) void sparse_offsets_kernel(const SparseArgs a)
{
    const int64_t nbnd = (int64_t)a.NB + 1;
    const int64_t wpc = (nbnd + 63) / 64; // waves per client
    const int64_t waves = (int64_t)a.K * wpc;
    const int lane = threadIdx.x & 63;
    for (int64_t w = global_tid() / 64; w < waves; w += grid_threads() / 64) {
        const int k = (int)(w / wpc);
        const int64_t b0 = (w % wpc) * 64;
        const int64_t b1 = min(b0 + 63, nbnd - 1);
        const int64_t *ix = a.idx[k];
        const int64_t n = a.nnz[k];
        const int64_t t0 = min(b0 * a.R, a.N), t1 = min(b1 * a.R, a.N);
        int64_t edge = 0;
        if (lane == 0)
            edge = sparse_lower_bound(ix, 0, n, t0, -1, a.N);
        else if (lane == 63)
            edge = sparse_lower_bound(ix, 0, n, t1, -1, a.N);
        const int64_t p0 = __shfl(edge, 0, 64), p1 = __shfl(edge, 63, 64);
        const int64_t b = b0 + lane;
        if (b > b1)
            continue;
        int64_t lo;
        if (b == b0)
            lo = p0;
        else if (b == b1)
            lo = p1;
        else
            lo = sparse_lower_bound(ix, p0, max(p0, p1), min(b * a.R, a.N), t0 - 1, t1);
        a.offs[(int64_t)k * nbnd + b] = lo;
        if ((b == 0 && lo > 0) || (b == a.NB && lo < n))
            *a.err = FA_ERR_INDEX;
    }
}

// One workgroup per parameter range of R = (whole tiles) parameters.  For
// each tile of SP_TILE parameters, LDS holds the fp32 sum and a bit mask of
// the clients that sent the parameter (MW 32-bit words: K <= 32 * MW); the
// weight sum W and the client count follow from the mask when the tile is
// finalized.  Clients are merged strictly in order, one barrier between
// client batches, so each parameter sees the same FMA order as the dense
// path; inside one batch the indices are unique, so lanes never collide on a
// sum and no float atomics are used (the mask bit is set with an LDS OR).
//
// A client's entries for the tile come as one coalesced batch of SP_THREADS
// (index, value) pairs read from its cursor; the batches of SP_GROUP clients
// are loaded together so their latencies overlap.  The in-tile entries of a
// sorted batch are a prefix: each wave counts its own with a ballot and the
// counts meet in LDS (double-buffered, so one barrier per batch suffices).
// The cursor advances by the count; a batch that lies wholly inside the tile
// loads the next one.  After the last client the tile is finalized and
// written once.
//
// Sortedness: each entry is checked against its predecessor -- the lane
// below it in the wave, the last lane of the wave before (exchanged in LDS
// with the counts), the last entry of the batch before, or at the range
// start the entry before the range, read once per workgroup -- and at the
// range's end every cursor must have reached its end offset.
//
// Eight waves per SIMD for the 256- and 512-lane tiles with one mask word
// (the measured configurations): the merge is bound by how many batches are
// in flight, and the scalar registers would otherwise cap residency at seven.
// Two mask words take more LDS than eight resident workgroups leave.
template <int MW, int SP_TILE, int SP_THREADS>
constexpr int sparse_min_blocks()
{
    return (MW == 1 && (SP_THREADS == 256 || SP_THREADS == 512)) ? 2048 / SP_THREADS : 1;
}

template <int MW, int SP_TILE, int SP_THREADS>
__global__ __launch_bounds__(SP_THREADS, (sparse_min_blocks<MW, SP_TILE, SP_THREADS>())) void
sparse_merge_kernel(const SparseArgs a)
{
    static_assert(SP_TILE == SP_THREADS * VEC, "one 8-parameter group per lane at finalize");
    constexpr int WAVES = SP_THREADS / 64;
    __shared__ __attribute__((aligned(16))) float s_acc[SP_TILE];
    __shared__ __attribute__((aligned(16))) uint32_t s_mask[MW][SP_TILE];
    __shared__ int64_t s_cur[FA_MAX_CLIENTS];
    __shared__ int64_t s_end[FA_MAX_CLIENTS];
    __shared__ uint32_t s_nk[FA_MAX_CLIENTS];
    __shared__ int64_t s_prev0[FA_MAX_CLIENTS];
    __shared__ int s_count[2][WAVES];
    __shared__ int64_t s_edge[2][WAVES];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int b = blockIdx.x;
    const int64_t r0 = (int64_t)b * a.R;
    const int64_t r1 = min(r0 + a.R, a.N);
    bool bad = false;
    int parity = 0;

    if (tid < a.K) {
        const int64_t c0 = a.offs[(int64_t)tid * (a.NB + 1) + b];
        int64_t c1 = a.offs[(int64_t)tid * (a.NB + 1) + b + 1];
        if (c1 < c0)
            bad = true; // offsets out of order: the list is not sorted
        c1 = max(c1, c0);
        s_cur[tid] = c0;
        s_end[tid] = min(c1, a.nnz[tid]);
        s_nk[tid] = a.wi[tid];
        // the entry before the range's first one, for the sortedness check
        s_prev0[tid] = c0 > 0 && c0 <= a.nnz[tid] ? a.idx[tid][c0 - 1] : -1;
    }
    for (int l = tid; l < SP_TILE; l += SP_THREADS) {
        s_acc[l] = 0.0f;
#pragma unroll
        for (int m = 0; m < MW; ++m)
            s_mask[m][l] = 0u;
    }
    __syncthreads();

    for (int64_t t0 = r0; t0 < r1; t0 += SP_TILE) {
        const int64_t t1 = min(t0 + SP_TILE, r1);
        for (int k0 = 0; k0 < a.K; k0 += SP_GROUP) {
            // one batch per client of the group: this lane's entry and its
            // value (INT64_MAX where the lane holds no entry)
            int64_t gix[SP_GROUP];
            float gval[SP_GROUP];
#pragma unroll
            for (int g = 0; g < SP_GROUP; ++g) {
                gix[g] = INT64_MAX;
                gval[g] = 0.0f;
                const int k = k0 + g;
                if (k < a.K) {
                    const int64_t p = s_cur[k] + tid;
                    if (p < s_end[k]) {
                        gix[g] = a.idx[k][p];
                        gval[g] = a.val[k][p];
                    }
                }
            }
#pragma unroll
            for (int g = 0; g < SP_GROUP; ++g) {
                const int k = k0 + g;
                if (k < a.K) {
                    int64_t p0 = s_cur[k];
                    const int64_t pend = s_end[k];
                    const float w = a.w[k];
                    const uint32_t bit = 1u << (k & 31);
                    uint32_t *mrow = s_mask[MW > 1 ? (k >> 5) : 0];
                    // One round: the batch's in-tile entries (a prefix) are
                    // counted by wave ballots that meet in LDS, checked
                    // against their predecessors and merged; returns the
                    // count, and the batch's last index through batch_last.
                    auto round = [&](int64_t ix, float val, int64_t first_prev, int64_t &batch_last) {
                        const bool in = ix < t1;
                        const uint64_t bal = __ballot(in);
                        const int64_t up = __shfl_up(ix, 1, 64);
                        if (lane == 0)
                            s_count[parity][wave] = __popcll(bal);
                        if (lane == 63)
                            s_edge[parity][wave] = ix;
                        __syncthreads();
                        int c = 0;
#pragma unroll
                        for (int v = 0; v < WAVES; ++v)
                            c += s_count[parity][v];
                        const int64_t prev =
                            lane > 0 ? up : (wave > 0 ? s_edge[parity][wave - 1] : first_prev);
                        batch_last = s_edge[parity][WAVES - 1];
                        parity ^= 1;
                        if (in) {
                            if (ix <= prev || ix < t0) {
                                bad = true;
                            } else {
                                const int l = (int)(ix - t0);
                                s_acc[l] = __builtin_fmaf(w, val, s_acc[l]);
                                atomicOr(&mrow[l], bit);
                            }
                        }
                        return c;
                    };
                    // index of the entry before this batch's first: before
                    // the range, the previous range's last entry; in later
                    // tiles the previous entry lies below t0, which the
                    // ix >= t0 test covers; after a refill, the last entry
                    // of the batch before
                    int64_t batch_last;
                    int c = round(gix[g], gval[g], t0 == r0 ? s_prev0[k] : -1, batch_last);
                    p0 += c;
                    // A whole batch inside the tile (rare at the default
                    // tile): read the next ones.  The refills live in their
                    // own loop so the group's batches keep their own,
                    // partial load waits.
                    if (c == SP_THREADS && p0 < pend) {
                        do {
                            const int64_t first_prev = batch_last;
                            const int64_t p = p0 + tid;
                            int64_t rix = INT64_MAX;
                            float rval = 0.0f;
                            if (p < pend) {
                                rix = a.idx[k][p];
                                rval = a.val[k][p];
                            }
                            c = round(rix, rval, first_prev, batch_last);
                            p0 += c;
                        } while (c == SP_THREADS && p0 < pend);
                    }
                    if (tid == 0)
                        s_cur[k] = p0;
                }
            }
        }
        __syncthreads();

        // finalize the tile: each lane takes the 4-parameter quads at 4 * tid
        // and SP_TILE / 2 + 4 * tid, so the 16-byte stores of a wave cover
        // whole cache lines
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int lq = h * (SP_TILE / 2) + tid * 4;
            const int64_t eq = t0 + lq;
            float acc[4];
            uint32_t W[4], cnt[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t wsum = 0, c = 0;
#pragma unroll
                for (int m = 0; m < MW; ++m) {
                    uint32_t bits = s_mask[m][lq + j];
                    c += __popc(bits);
                    while (bits) {
                        wsum += s_nk[m * 32 + __ffs(bits) - 1];
                        bits &= bits - 1;
                    }
                    s_mask[m][lq + j] = 0u;
                }
                W[j] = wsum;
                cnt[j] = c;
                acc[j] = s_acc[lq + j];
                s_acc[lq + j] = 0.0f;
            }
            if (a.aligned && eq + 4 <= t1) {
                // through buffers over the tile's part of each array (nt
                // loads, sc1 nt stores)
                const int64_t tn = t1 - t0;
                const f32x4 bq = bio<DT_F32>::q(span_rsrc(a.base + t0, tn * 4), lq * 4);
                const float b4[4] = {bq.x, bq.y, bq.z, bq.w};
                float r[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (W[j] > 0) {
                        const float q = acc[j] / (a.zero_fill ? a.S_all : (float)W[j]);
                        r[j] = a.mode == MODE_DELTAS ? b4[j] + q : q;
                    } else {
                        r[j] = b4[j];
                    }
                }
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{r[0], r[1], r[2], r[3]}),
                                                       span_rsrc(a.out + t0, tn * 4), lq * 4, 0, BUF_STORE);
                if (a.counts) {
                    if (a.counts_u32)
                        __builtin_amdgcn_raw_buffer_store_b128(
                            u32x4{cnt[0], cnt[1], cnt[2], cnt[3]},
                            span_rsrc(static_cast<uint32_t *>(a.counts) + t0, tn * 4), lq * 4, 0, BUF_STORE);
                    else
                        __builtin_amdgcn_raw_buffer_store_b32(
                            cnt[0] | (cnt[1] << 8) | (cnt[2] << 16) | (cnt[3] << 24),
                            span_rsrc(static_cast<uint8_t *>(a.counts) + t0, tn), lq, 0, BUF_STORE);
                }
                if (a.wsum)
                    __builtin_amdgcn_raw_buffer_store_b128(u32x4{W[0], W[1], W[2], W[3]},
                                                           span_rsrc(a.wsum + t0, tn * 4), lq * 4, 0, BUF_STORE);
            } else {
                for (int j = 0; j < 4; ++j) {
                    const int64_t e = eq + j;
                    if (e < t1) {
                        const float bv = a.base[e];
                        float r = bv;
                        if (W[j] > 0) {
                            const float q = acc[j] / (a.zero_fill ? a.S_all : (float)W[j]);
                            r = a.mode == MODE_DELTAS ? bv + q : q;
                        }
                        a.out[e] = r;
                        if (a.counts) {
                            if (a.counts_u32)
                                static_cast<uint32_t *>(a.counts)[e] = cnt[j];
                            else
                                static_cast<uint8_t *>(a.counts)[e] = (uint8_t)cnt[j];
                        }
                        if (a.wsum)
                            a.wsum[e] = W[j];
                    }
                }
            }
        }
        // the next tile's first barrier orders these zeroes before use
    }
    // every entry between the range's offsets lies inside the range when the
    // list is sorted, so each cursor has reached its end; entries left over
    // mean the list is out of order (the tile loop's barriers order the last
    // cursor update before this read)
    if (tid < a.K && s_cur[tid] != s_end[tid])
        bad = true;
    if (bad)
        *a.err = FA_ERR_INDEX;
}

// ================================================================ tiled index accumulate

// Client-at-a-time sparse accumulate over dense tiles.  A client's list of
// about one parameter in 16 or more touches nearly every cache line of the
// accumulator's fp32 sums, weight sums and counts, so scattered updates move
// whole lines anyway, as read-modify-writes interleaved at random; reading
// and writing the tiles that hold the list as whole streams costs about as
// many bytes in long runs instead.
//
// The tiled path needs a sorted list inside the accumulator: a first kernel
// checks it and sets *gate when it is not, and the tiled kernel then leaves
// the call to the scatter kernel, which reports and skips the bad entries.
__global__ __launch_bounds__(256) void stream_index_check_kernel(const StreamArgs a, int *gate)
{
    const int64_t span = a.N - a.offset;
    bool bad = false;
    for (int64_t j = global_tid(); j < a.len; j += grid_threads()) {
        const int64_t ix = a.idx[j];
        const int64_t prev = j > 0 ? a.idx[j - 1] : -1;
        bad = bad || ix < 0 || ix >= span || ix <= prev;
    }
    if (__ballot(bad) != 0 && (threadIdx.x & 63) == 0)
        *gate = 1;
}

// A form with one 16-byte load per lane for two entries (the entry before
// them from the lane below) ran slower: 3.16 against 3.10 ms per client
// with the tiles.

// Each workgroup takes tpw consecutive tiles of IT_TILE parameters,
// tiles aligned to the accumulator, counted from the one holding the list's
// first parameter up to the one holding its last.  Per tile, each lane reads
// the sums, weight sums and counts of its two 4-parameter quads (at 4 tid and
// half a tile further: whole-line accesses); the tile's entries, consecutive
// in the sorted list, arrive in batches of 256 from the list cursor (the
// in-tile ones are a prefix, counted by wave ballots) and are scattered into
// LDS as a value and a presence bit; then each lane applies its present
// parameters with the scatter kernel's operations (acc = fma(n_k, x, acc),
// wsum += n_k, count += 1) and writes its quads back.  A 64-byte run of sums
// (or weight sums) that no entry touched, four lanes' quads, is not written.
//
// One tile per workgroup (tpw, the tiles per workgroup, is 1 below 2^35
// parameters) and 7 resident workgroups per CU, measured on a
// 10^8-entry client of a 10^9-parameter accumulator (ms per client with the
// check): tiles per workgroup 1, 2, 4, 8 at no cap 3.44, 3.53, 3.58, 3.66;
// one tile at caps of 4, 5, 6, 7, 8 workgroups per CU 3.74, 3.75, 3.29,
// 3.10, 3.44.  Requesting the next tile's batch and quads while the current
// tile is applied (two register sets, every load through a range-bounded
// buffer so none sat under a branch) ran no faster: 3.74-3.79 against 3.78
// ms at 4 tiles per workgroup.
constexpr int IT_RESIDENT = 7;

template <int DT>
__global__ __launch_bounds__(256) void stream_acc_index_tile_kernel(const StreamArgs a, const int *gate,
                                                                    int64_t tpw)
{
    __shared__ float s_val[IT_TILE];
    __shared__ uint32_t s_bit[IT_TILE / 32];
    __shared__ int s_count[2][4];
    __shared__ int64_t s_p;
    if (*gate != 0 || a.len == 0)
        return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // the list's ends, as parameters of the accumulator (the list is sorted)
    const int64_t first = a.offset + a.idx[0];
    const int64_t last = a.offset + a.idx[a.len - 1];
    const int64_t tb = first / IT_TILE + (int64_t)blockIdx.x * tpw;
    const int64_t tl = last / IT_TILE;
    if (tb > tl)
        return;
    const int64_t te = min(tb + tpw, tl + 1);
    if (tid < IT_TILE / 32)
        s_bit[tid] = 0u;
    if (tid == 0)
        s_p = blockIdx.x == 0 ? 0
                              : sparse_lower_bound(a.idx, 0, a.len, tb * IT_TILE - a.offset, -1, a.N - a.offset);
    __syncthreads();
    int64_t p = s_p;
    int parity = 0;
    const int q0 = tid * 4, q1 = IT_TILE / 2 + tid * 4;
    for (int64_t t = tb; t < te; ++t) {
        const int64_t t0 = t * IT_TILE, t1 = t0 + IT_TILE;
        const int64_t tn = min((int64_t)IT_TILE, a.N - t0);
        const auto ra = span_rsrc(a.acc + t0, tn * 4);
        const auto rw = span_rsrc(a.wsum + t0, tn * 4);
        const auto rc = span_rsrc(a.count ? a.count + t0 : nullptr, a.count ? tn : 0);
        uint32_t n0 = __builtin_amdgcn_raw_buffer_load_b32(rc, q0, 0, BUF_NT);
        uint32_t n1 = __builtin_amdgcn_raw_buffer_load_b32(rc, q1, 0, BUF_NT);
        int c;
        do {
            const int64_t q = p + tid;
            int64_t ix = INT64_MAX;
            float v = 0.0f;
            if (q < a.len) {
                ix = a.offset + a.idx[q];
                v = io<DT>::load1(a.chunk, q);
            }
            const bool in = ix < t1;
            const uint64_t bal = __ballot(in);
            if (lane == 0)
                s_count[parity][wave] = __popcll(bal);
            __syncthreads();
            c = s_count[parity][0] + s_count[parity][1] + s_count[parity][2] + s_count[parity][3];
            parity ^= 1;
            if (in) {
                const int l = (int)(ix - t0);
                s_val[l] = v;
                atomicOr(&s_bit[l >> 5], 1u << (l & 31));
            }
            p += c;
        } while (c == 256 && p < a.len);
        __syncthreads();
        const uint32_t b0 = (s_bit[q0 >> 5] >> (q0 & 31)) & 15u;
        const uint32_t b1 = (s_bit[q1 >> 5] >> (q1 & 31)) & 15u;
        // 16 parameters (four lanes' quads) share a 64-byte run
        const bool t0run = (s_bit[q0 >> 5] >> (q0 & 16)) & 0xFFFFu;
        const bool t1run = (s_bit[q1 >> 5] >> (q1 & 16)) & 0xFFFFu;
        f32x4 c0 = {0, 0, 0, 0}, c1 = {0, 0, 0, 0};
        u32x4 w0 = {0, 0, 0, 0}, w1 = {0, 0, 0, 0};
        if (t0run) {
            c0 = bio<DT_F32>::q(ra, q0 * 4);
            w0 = __builtin_amdgcn_raw_buffer_load_b128(rw, q0 * 4, 0, BUF_NT);
        }
        if (t1run) {
            c1 = bio<DT_F32>::q(ra, q1 * 4);
            w1 = __builtin_amdgcn_raw_buffer_load_b128(rw, q1 * 4, 0, BUF_NT);
        }
        float x0[4] = {c0.x, c0.y, c0.z, c0.w}, x1[4] = {c1.x, c1.y, c1.z, c1.w};
        uint32_t y0[4] = {w0.x, w0.y, w0.z, w0.w}, y1[4] = {w1.x, w1.y, w1.z, w1.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if ((b0 >> j) & 1u) {
                x0[j] = __builtin_fmaf(a.w, s_val[q0 + j], x0[j]);
                y0[j] += a.wi;
                n0 += 1u << (8 * j);
            }
            if ((b1 >> j) & 1u) {
                x1[j] = __builtin_fmaf(a.w, s_val[q1 + j], x1[j]);
                y1[j] += a.wi;
                n1 += 1u << (8 * j);
            }
        }
        if (t0run) {
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{x0[0], x0[1], x0[2], x0[3]}),
                                                   ra, q0 * 4, 0, BUF_STORE);
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{y0[0], y0[1], y0[2], y0[3]}, rw, q0 * 4, 0, BUF_STORE);
        }
        if (t1run) {
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{x1[0], x1[1], x1[2], x1[3]}),
                                                   ra, q1 * 4, 0, BUF_STORE);
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{y1[0], y1[1], y1[2], y1[3]}, rw, q1 * 4, 0, BUF_STORE);
        }
        __builtin_amdgcn_raw_buffer_store_b32(n0, rc, q0, 0, BUF_STORE);
        __builtin_amdgcn_raw_buffer_store_b32(n1, rc, q1, 0, BUF_STORE);
        __syncthreads(); // every lane has read the tile's bits and values
        if (tid < IT_TILE / 32)
            s_bit[tid] = 0u;
        // the next tile's first batch barrier orders these zeroes before its scatter
    }
}

// ================================================================ checksum

__device__ __forceinline__ uint64_t fmix64(uint64_t k)
{
    k ^= k >> 33;
    k *= 0xff51afd7ed558ccdull;
    k ^= k >> 33;
    k *= 0xc4ceb9fe1a85ec53ull;
    k ^= k >> 33;
    return k;
}

__device__ __forceinline__ uint64_t elem_hash(int64_t i, uint32_t bits)
{
    return fmix64(((uint64_t)i * 0x9E3779B97F4A7C15ull) ^ (uint64_t)bits);
}

// The hashes of one 16-byte vector starting at element e0: 4 fp32 or 8 bf16.
// The index products i * 0x9E37... step by one addition (mod 2^64).
template <int DT> __device__ __forceinline__ uint64_t vec_hash(const u32x4 &r, int64_t e0)
{
    constexpr uint64_t G = 0x9E3779B97F4A7C15ull;
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
    uint64_t m = (uint64_t)e0 * G;
    uint64_t h = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if constexpr (DT == DT_F32) {
            h += fmix64(m ^ (uint64_t)w[j]);
            m += G;
        } else {
            h += fmix64(m ^ (uint64_t)(w[j] & 0xFFFFu));
            m += G;
            h += fmix64(m ^ (uint64_t)(w[j] >> 16));
            m += G;
        }
    }
    return h;
}

// Integer sum of per-element hashes: exact and independent of the order the
// lanes add in.  16-byte vectors, four issued per step, then the elements
// past the last whole vector; lanes reduce across the wavefront with
// butterfly shuffles, the four wavefronts through LDS, then one 64-bit
// atomic add per workgroup.
template <int DT>
__global__ __launch_bounds__(256) void checksum_kernel(const void *buf, int64_t count, bool aligned,
                                                       unsigned long long *out)
{
    constexpr int EPV = DT == DT_F32 ? 4 : 8;
    const int64_t nvec = aligned ? count / EPV : 0;
    const u32x4 *vp = static_cast<const u32x4 *>(buf);
    const int64_t stride = grid_threads();
    uint64_t h = 0;
    int64_t v = global_tid();
    for (; v + 3 * stride < nvec; v += 4 * stride) {
        u32x4 r[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            r[u] = __builtin_nontemporal_load(vp + v + u * stride);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            h += vec_hash<DT>(r[u], (v + u * stride) * EPV);
    }
    for (; v < nvec; v += stride)
        h += vec_hash<DT>(__builtin_nontemporal_load(vp + v), v * EPV);
    for (int64_t i = nvec * EPV + global_tid(); i < count; i += stride) {
        const uint32_t bits = DT == DT_F32 ? static_cast<const uint32_t *>(buf)[i]
                                           : (uint32_t) static_cast<const uint16_t *>(buf)[i];
        h += elem_hash(i, bits);
    }
    __shared__ unsigned long long wh[4];
    unsigned long long r = h;
    for (int off = 32; off > 0; off >>= 1)
        r += __shfl_xor(r, off);
    if ((threadIdx.x & 63) == 0)
        wh[threadIdx.x >> 6] = r;
    __syncthreads();
    if (threadIdx.x == 0)
        atomicAdd(out, wh[0] + wh[1] + wh[2] + wh[3]);
}

// fp64 sum of a value from each of the 64 lanes by a butterfly.  Lanes i and
// i^off add the same two values (in either order, which IEEE addition does
// not see), so every lane ends with the same sum and the pairing is fixed.
__device__ __forceinline__ double wave_sum_f64(double v)
{
    for (int off = 32; off > 0; off >>= 1)
        v += __shfl_xor(v, off);
    return v;
}

template <int DT> __device__ __forceinline__ double elem_value(uint32_t bits)
{
    return DT == DT_F32 ? (double)__uint_as_float(bits) : (double)__uint_as_float(bits << 16);
}

// Hash and fp64 value sum in one read.  The order of the additions is set by
// the element count alone (not by the grid, the alignment or the device), so
// the sum is the same bits on every call: tiles of SUM_TILE elements; in a
// tile, thread j adds, from +0 and in element order, the elements of the
// 16-byte vectors j, j + 256, ... of the tile (fp32: 8 vectors of 4, bf16: 4
// of 8); the thread sums meet in a butterfly per wavefront and the four
// wavefront sums as (w0 + w1) + (w2 + w3), giving part[t].  Tiles wholly
// inside an aligned buffer are read as vectors, the rest element by element
// in the same order.
template <int DT, bool HASH>
__global__ __launch_bounds__(256) void checksum_sum_kernel(const void *buf, int64_t count,
                                                           bool aligned,
                                                           unsigned long long *hash, double *part)
{
    constexpr int EPV = DT == DT_F32 ? 4 : 8;
    constexpr int VPT = SUM_TILE / EPV; // vectors per tile
    constexpr int RV = VPT / 256;       // vectors per thread and tile
    const int64_t T = (count + SUM_TILE - 1) / SUM_TILE;
    const int64_t full = aligned ? count / SUM_TILE : 0;
    const int j = threadIdx.x;
    __shared__ double wsum[4];
    uint64_t h = 0;
    for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
        double s = 0.0;
        if (t < full) {
            // with the hash, GV vectors at a time: its 64-bit products would
            // otherwise hold enough registers to cut the waves per SIMD
            constexpr int GV = HASH ? (DT == DT_F32 ? 4 : 2) : RV;
            const u32x4 *vp = static_cast<const u32x4 *>(buf) + t * VPT + j;
#pragma unroll 1
            for (int u0 = 0; u0 < RV; u0 += GV) {
                u32x4 r[GV];
#pragma unroll
                for (int u = 0; u < GV; ++u)
                    r[u] = __builtin_nontemporal_load(vp + (u0 + u) * 256);
#pragma unroll
                for (int u = 0; u < GV; ++u) {
                    const uint32_t w[4] = {r[u].x, r[u].y, r[u].z, r[u].w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if constexpr (DT == DT_F32) {
                            s += elem_value<DT>(w[q]);
                        } else {
                            s += elem_value<DT>(w[q] & 0xFFFFu);
                            s += elem_value<DT>(w[q] >> 16);
                        }
                    }
                    if constexpr (HASH)
                        h += vec_hash<DT>(r[u], (t * VPT + (u0 + u) * 256 + j) * EPV);
                }
            }
        } else {
            for (int u = 0; u < RV; ++u)
                for (int c = 0; c < EPV; ++c) {
                    const int64_t e = t * SUM_TILE + (int64_t)(u * 256 + j) * EPV + c;
                    if (e >= count)
                        break;
                    const uint32_t bits = DT == DT_F32
                                              ? static_cast<const uint32_t *>(buf)[e]
                                              : (uint32_t) static_cast<const uint16_t *>(buf)[e];
                    s += elem_value<DT>(bits);
                    if constexpr (HASH)
                        h += elem_hash(e, bits);
                }
        }
        s = wave_sum_f64(s);
        if ((j & 63) == 0)
            wsum[j >> 6] = s;
        __syncthreads();
        if (j == 0)
            part[t] = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
        __syncthreads();
    }
    if constexpr (HASH) {
        // one atomic per workgroup: they all land on one word
        __shared__ unsigned long long wh[4];
        unsigned long long r = h;
        for (int off = 32; off > 0; off >>= 1)
            r += __shfl_xor(r, off);
        if ((j & 63) == 0)
            wh[j >> 6] = r;
        __syncthreads();
        if (j == 0)
            atomicAdd(hash, wh[0] + wh[1] + wh[2] + wh[3]);
    }
}

// The tile sums' total, in a fixed order: thread j adds part[j], part[j +
// 1024], ... from +0, then a butterfly per wavefront, then the 16 wavefront
// sums pairwise ((w0 + w1) + (w2 + w3)) + ... .  T = 0 gives +0.
__global__ __launch_bounds__(SUM_FINISH_THREADS) void sum_finish_kernel(const double *part,
                                                                        int64_t T, double *out)
{
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < T; i += SUM_FINISH_THREADS)
        s += part[i];
    s = wave_sum_f64(s);
    __shared__ double w[SUM_FINISH_THREADS / 64];
    if ((threadIdx.x & 63) == 0)
        w[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        double v[SUM_FINISH_THREADS / 64];
        for (int i = 0; i < SUM_FINISH_THREADS / 64; ++i)
            v[i] = w[i];
        for (int n = SUM_FINISH_THREADS / 64; n > 1; n >>= 1)
            for (int i = 0; i < n / 2; ++i)
                v[i] = v[2 * i] + v[2 * i + 1];
        *out = v[0];
    }
}

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t *p, int64_t words, uint32_t value)
{
    for (int64_t i = global_tid(); i < words; i += grid_threads())
        p[i] = value;
}

__global__ __launch_bounds__(64) void fill_u8_kernel(uint8_t *p, int64_t bytes, uint8_t value)
{
    for (int64_t i = global_tid(); i < bytes; i += grid_threads())
        p[i] = value;
}

// Element copy with type conversion (round-to-nearest-even when narrowing):
// the result when no client contributed at all.
template <int SDT, int DDT>
__global__ __launch_bounds__(256) void convert_kernel(const void *src, void *dst, int64_t N)
{
    for (int64_t e = global_tid(); e < N; e += grid_threads())
        io<DDT>::store1(dst, e, io<SDT>::load1(src, e));
}

// ================================================================ launchers

static inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

static int lds_bytes_per_cu()
{
    // per device, filled on first use; threads that race store the same value
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
                hipSuccess ||
            v <= 0)
            v = 65536;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

// Streaming kernels over HBM run fastest with few resident waves per CU (a
// measured property of MI355X when reads and writes mix: more waves in
// flight only add DRAM read/write turnarounds).  Residency is capped by
// reserving dynamic LDS: a workgroup's LDS (its own plus the request)
// between 1/(cap+1) and 1/cap of the CU's LDS admits exactly `cap`
// workgroups per CU.  The kernels do not use the request.
template <typename F>
static size_t residency_lds(F *kernel, int cap)
{
    if (cap <= 0)
        return 0;
    const int lds = lds_bytes_per_cu();
    if (lds <= 0)
        return 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 0;
    // per kernel and device: the kernel's own LDS, and the largest request
    // allowed so far
    struct Entry {
        size_t own = 0, allowed = 0;
        bool known = false;
    };
    static std::mutex mu;
    static std::map<std::pair<const void *, int>, Entry> table;
    const void *fn = reinterpret_cast<const void *>(kernel);
    std::lock_guard<std::mutex> lock(mu);
    Entry &en = table[{fn, dev}];
    if (!en.known) {
        hipFuncAttributes attr;
        if (hipFuncGetAttributes(&attr, fn) != hipSuccess) {
            (void)hipGetLastError();
            return 0;
        }
        en.own = attr.sharedSizeBytes;
        en.known = true;
    }
    const size_t total = ((size_t)lds / cap + (size_t)lds / (cap + 1)) / 2;
    if (total <= en.own)
        return 0;
    const size_t bytes = total - en.own;
    if (bytes > en.allowed) {
        if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) != hipSuccess) {
            (void)hipGetLastError();
            return 0;
        }
        en.allowed = bytes;
    }
    return bytes;
}

// Workgroups for `work` items, `threads` per workgroup, at most `cap` (0: no
// cap).  A launch holds at most 2^32 - 1 work-items per dimension, so with
// the 256-lane workgroups every launch through here uses, the grid stops at
// MAX_GRID_256; the kernels walk their work grid-stride and cover the rest.
constexpr int64_t MAX_GRID_256 = 0xFFFFFFFFll / 256;

static inline unsigned grid_for(int64_t work, int threads, int64_t cap)
{
    int64_t g = ceil_div(work, threads);
    if (cap > 0 && g > cap)
        g = cap;
    if (g < 1)
        g = 1;
    if (g > MAX_GRID_256)
        g = MAX_GRID_256;
    return (unsigned)g;
}

template <int XDT, int ODT, int BDT, int MODE, int KC>
static void dense_vec_launch(const DenseArgs &a, int64_t nvec, int64_t cap, int resident, hipStream_t s)
{
    auto *k = &dense_vec_kernel<XDT, ODT, BDT, MODE, KC>;
    k<<<grid_for(nvec, 256, cap), 256, residency_lds(k, resident), s>>>(a, nvec);
}

template <int XDT, int ODT, int BDT, int MODE>
static hipError_t dense_launch_t(const DenseArgs &a, bool aligned, int64_t cap, int resident,
                                 hipStream_t s)
{
    const int64_t nvec = aligned ? a.N / VEC : 0;
    if (nvec > 0) {
        // Fixed client counts get kernels of their own; other counts load
        // their clients in batches, of 16 once there are more than 16 (one
        // batch boundary fewer per 16 clients: 2-3% at K = 20 ... 64, where
        // dedicated K = 32 or 64 kernels need up to 256 VGPRs and run slower).
        switch (a.K) {
        case 3: dense_vec_launch<XDT, ODT, BDT, MODE, 3>(a, nvec, cap, resident, s); break;
        case 8: dense_vec_launch<XDT, ODT, BDT, MODE, 8>(a, nvec, cap, resident, s); break;
        case 16: dense_vec_launch<XDT, ODT, BDT, MODE, 16>(a, nvec, cap, resident, s); break;
        default:
            if (a.K > 16)
                dense_vec_launch<XDT, ODT, BDT, MODE, -16>(a, nvec, cap, resident, s);
            else
                dense_vec_launch<XDT, ODT, BDT, MODE, -8>(a, nvec, cap, resident, s);
            break;
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    const int64_t first = nvec * VEC;
    const int64_t rest = a.N - first;
    if (rest > 0) {
        dense_scalar_kernel<XDT, ODT, BDT, MODE><<<grid_for(rest, 256, cap), 256, 0, s>>>(a, first, rest);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <template <int, int, int, int> class F, typename... Args>
static hipError_t dispatch4(int xdt, int odt, int bdt, int mode, Args &&...args)
{
    // 2 x 2 x 2 x 2 instantiations
#define FA_CASE(X, O, B, M)                                                                        \
    if (xdt == X && odt == O && bdt == B && mode == M)                                            \
        return F<X, O, B, M>::run(args...);
    FA_CASE(DT_F32, DT_F32, DT_F32, MODE_WEIGHTS)
    FA_CASE(DT_F32, DT_F32, DT_F32, MODE_DELTAS)
    FA_CASE(DT_F32, DT_F32, DT_BF16, MODE_WEIGHTS)
    FA_CASE(DT_F32, DT_F32, DT_BF16, MODE_DELTAS)
    FA_CASE(DT_F32, DT_BF16, DT_F32, MODE_WEIGHTS)
    FA_CASE(DT_F32, DT_BF16, DT_F32, MODE_DELTAS)
    FA_CASE(DT_F32, DT_BF16, DT_BF16, MODE_WEIGHTS)
    FA_CASE(DT_F32, DT_BF16, DT_BF16, MODE_DELTAS)
    FA_CASE(DT_BF16, DT_F32, DT_F32, MODE_WEIGHTS)
    FA_CASE(DT_BF16, DT_F32, DT_F32, MODE_DELTAS)
    FA_CASE(DT_BF16, DT_F32, DT_BF16, MODE_WEIGHTS)
    FA_CASE(DT_BF16, DT_F32, DT_BF16, MODE_DELTAS)
    FA_CASE(DT_BF16, DT_BF16, DT_F32, MODE_WEIGHTS)
    FA_CASE(DT_BF16, DT_BF16, DT_F32, MODE_DELTAS)
    FA_CASE(DT_BF16, DT_BF16, DT_BF16, MODE_WEIGHTS)
    FA_CASE(DT_BF16, DT_BF16, DT_BF16, MODE_DELTAS)
#undef FA_CASE
    return hipErrorInvalidValue;
}

template <int X, int O, int B, int M> struct DenseRun {
    static hipError_t run(const DenseArgs &a, bool aligned, int64_t cap, int resident, hipStream_t s)
    {
        return dense_launch_t<X, O, B, M>(a, aligned, cap, resident, s);
    }
};

template <int X, int O, int B, int M> struct MaskedRun {
    static hipError_t run(const MaskedArgs &a, bool aligned, hipStream_t s)
    {
        if (aligned) {
            const int64_t nvec_all = ceil_div(a.N, VEC);
            // the windowed kernel takes one run of vpb vectors per workgroup:
            // runs long enough that their workgroups fit one launch
            MaskedArgs b = a;
            if (ceil_div(nvec_all, b.vpb) > MAX_GRID_256)
                b.vpb = ceil_div(nvec_all, MAX_GRID_256);
            const unsigned g = grid_for(nvec_all, (int)b.vpb, 0);
            if (b.T <= TAB_SEGS)
                masked_table_kernel<X, O, B, M, 1><<<g, 256, 0, s>>>(b);
            else
                masked_vec_kernel<X, O, B, M><<<g, 256, 0, s>>>(b);
        } else {
            masked_scalar_kernel<X, O, B, M><<<grid_for(a.N, 256, 65536), 256, 0, s>>>(a);
        }
        return hipGetLastError();
    }
};

hipError_t launch_dense(const DenseArgs &a, int xdt, int odt, int bdt, int mode, bool aligned,
                        int64_t grid_cap, int resident, hipStream_t s)
{
    return dispatch4<DenseRun>(xdt, odt, bdt, mode, a, aligned, grid_cap, resident, s);
}

hipError_t launch_masked(const MaskedArgs &a, int xdt, int odt, int bdt, int mode, bool aligned,
                         hipStream_t s)
{
    return dispatch4<MaskedRun>(xdt, odt, bdt, mode, a, aligned, s);
}

template <int DT, int PART>
static hipError_t stream_acc_t(const StreamArgs &a, bool aligned, int64_t cap, int resident,
                               hipStream_t s)
{
    const int64_t nvec = aligned ? a.len / VEC : 0;
    if (nvec > 0) {
        auto *k = &stream_acc_vec_kernel<DT, PART>;
        k<<<grid_for(nvec, 256, cap), 256, residency_lds(k, resident), s>>>(a, nvec);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    const int64_t first = nvec * VEC;
    const int64_t rest = a.len - first;
    if (rest > 0) {
        stream_acc_scalar_kernel<DT, PART><<<grid_for(rest, 256, cap), 256, 0, s>>>(a, first, rest);
        return hipGetLastError();
    }
    return hipSuccess;
}

hipError_t launch_stream_accumulate(const StreamArgs &a, int dt, int part, bool aligned,
                                    int64_t cap, int resident, hipStream_t s)
{
#define FA_CASE(D, P)                                                                              \
    if (dt == D && part == P)                                                                      \
        return stream_acc_t<D, P>(a, aligned, cap, resident, s);
    FA_CASE(DT_F32, PART_DENSE)
    FA_CASE(DT_F32, PART_RANGE)
    FA_CASE(DT_F32, PART_MASK)
    FA_CASE(DT_BF16, PART_DENSE)
    FA_CASE(DT_BF16, PART_RANGE)
    FA_CASE(DT_BF16, PART_MASK)
#undef FA_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_stream_accumulate_indices(const StreamArgs &a, int dt, bool tiled, int *gate, hipStream_t s)
{
    const unsigned g = grid_for(a.len, 256, 65536);
    if (!tiled) {
        StreamArgs b = a;
        b.gate = nullptr;
        if (dt == DT_F32)
            stream_acc_index_kernel<DT_F32><<<g, 256, 0, s>>>(b);
        else
            stream_acc_index_kernel<DT_BF16><<<g, 256, 0, s>>>(b);
        return hipGetLastError();
    }
    fill_u32_kernel<<<1, 64, 0, s>>>(reinterpret_cast<uint32_t *>(gate), 1, 0u);
    stream_index_check_kernel<<<g, 256, 0, s>>>(a, gate);
    // tiles from the list's first parameter to its last: at most this many;
    // one per workgroup, or consecutive runs of them where a grid of one per
    // workgroup would exceed the dispatch limit (accumulators beyond 2^35
    // parameters)
    const int64_t tiles = (a.N - a.offset) / IT_TILE + 2;
    const unsigned gt = grid_for(tiles, 1, 0);
    const int64_t tpw = ceil_div(tiles, (int64_t)gt);
    if (dt == DT_F32) {
        auto *k = &stream_acc_index_tile_kernel<DT_F32>;
        k<<<gt, 256, residency_lds(k, IT_RESIDENT), s>>>(a, gate, tpw);
    } else {
        auto *k = &stream_acc_index_tile_kernel<DT_BF16>;
        k<<<gt, 256, residency_lds(k, IT_RESIDENT), s>>>(a, gate, tpw);
    }
    // the scatter kernel runs only for a list the check refused: few
    // workgroups, each striding over the list
    StreamArgs b = a;
    b.gate = gate;
    const unsigned gs = g < 2048u ? g : 2048u;
    if (dt == DT_F32)
        stream_acc_index_kernel<DT_F32><<<gs, 256, 0, s>>>(b);
    else
        stream_acc_index_kernel<DT_BF16><<<gs, 256, 0, s>>>(b);
    return hipGetLastError();
}

template <int PARTIAL>
static hipError_t merge_t(const StreamArgs &a, bool aligned, int64_t cap, int resident, hipStream_t s)
{
    const int64_t nvec = aligned ? a.len / VEC : 0;
    if (nvec > 0) {
        auto *k = &stream_merge_vec_kernel<PARTIAL>;
        k<<<grid_for(nvec, 256, cap), 256, residency_lds(k, resident), s>>>(a, nvec);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    const int64_t first = nvec * VEC;
    const int64_t rest = a.len - first;
    if (rest > 0) {
        stream_merge_scalar_kernel<PARTIAL><<<grid_for(rest, 256, cap), 256, 0, s>>>(a, first, rest);
        return hipGetLastError();
    }
    return hipSuccess;
}

hipError_t launch_stream_merge(const StreamArgs &a, bool partial, bool aligned, int64_t cap,
                               int resident, hipStream_t s)
{
    return partial ? merge_t<1>(a, aligned, cap, resident, s) : merge_t<0>(a, aligned, cap, resident, s);
}

template <int B, int O, int M, int P>
static hipError_t finalize_t(const FinalizeArgs &a, bool aligned, int64_t cap, int resident,
                             hipStream_t s)
{
    const int64_t nvec = aligned ? a.N / VEC : 0;
    if (nvec > 0) {
        auto *k = &stream_finalize_vec_kernel<B, O, M, P>;
        k<<<grid_for(nvec, 256, cap), 256, residency_lds(k, resident), s>>>(a, nvec);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    const int64_t first = nvec * VEC;
    const int64_t rest = a.N - first;
    if (rest > 0) {
        stream_finalize_scalar_kernel<B, O, M, P><<<grid_for(rest, 256, cap), 256, 0, s>>>(a, first, rest);
        return hipGetLastError();
    }
    return hipSuccess;
}

hipError_t launch_stream_finalize(const FinalizeArgs &a, int bdt, int odt, int mode, int partial,
                                  bool aligned, int64_t cap, int resident, hipStream_t s)
{
#define FA_CASE(B, O, M, P)                                                                        \
    if (bdt == B && odt == O && mode == M && partial == P)                                        \
        return finalize_t<B, O, M, P>(a, aligned, cap, resident, s);
#define FA_CASES(B, O)                                                                             \
    FA_CASE(B, O, MODE_WEIGHTS, 0)                                                                 \
    FA_CASE(B, O, MODE_WEIGHTS, 1)                                                                 \
    FA_CASE(B, O, MODE_DELTAS, 0)                                                                  \
    FA_CASE(B, O, MODE_DELTAS, 1)
    FA_CASES(DT_F32, DT_F32)
    FA_CASES(DT_F32, DT_BF16)
    FA_CASES(DT_BF16, DT_F32)
    FA_CASES(DT_BF16, DT_BF16)
#undef FA_CASES
#undef FA_CASE
    return hipErrorInvalidValue;
}

template <int TILE, int THREADS> static int resident_blocks()
{
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, sparse_merge_kernel<1, TILE, THREADS>,
                                                     THREADS, 0) != hipSuccess ||
        occ <= 0) {
        (void)hipGetLastError();
        occ = 1;
    }
    return occ;
}

int sparse_resident_blocks_per_cu(int tile)
{
    switch (tile) {
    case 512: return resident_blocks<512, 64>();
    case 1024: return resident_blocks<1024, 128>();
    case 2048: return resident_blocks<2048, 256>();
    case 8192: return resident_blocks<8192, 1024>();
    default: return resident_blocks<4096, 512>();
    }
}

template <int TILE, int THREADS> static void merge_launch(const SparseArgs &a, hipStream_t s)
{
    if (a.K <= 32)
        sparse_merge_kernel<1, TILE, THREADS><<<a.NB, THREADS, 0, s>>>(a);
    else
        sparse_merge_kernel<2, TILE, THREADS><<<a.NB, THREADS, 0, s>>>(a);
}

hipError_t launch_sparse(const SparseArgs &a, hipStream_t s)
{
    const int64_t lanes = (int64_t)a.K * (((int64_t)a.NB + 64) / 64) * 64;
    sparse_offsets_kernel<<<grid_for(lanes, 256, 0), 256, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    switch (a.tile) {
    case 512: merge_launch<512, 64>(a, s); break;
    case 1024: merge_launch<1024, 128>(a, s); break;
    case 2048: merge_launch<2048, 256>(a, s); break;
    case 8192: merge_launch<8192, 1024>(a, s); break;
    default: merge_launch<4096, 512>(a, s); break;
    }
    return hipGetLastError();
}

hipError_t launch_checksum(const void *buf, int64_t count, int dt, uint64_t *hash, hipStream_t s)
{
    fill_u32_kernel<<<1, 64, 0, s>>>(reinterpret_cast<uint32_t *>(hash), 2, 0u);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || count == 0)
        return e;
    const bool aligned = (reinterpret_cast<uintptr_t>(buf) & 15u) == 0;
    const int epv = dt == DT_F32 ? 4 : 8;
    const unsigned g = grid_for(aligned ? ceil_div(count, epv) : count, 256, 4096);
    if (dt == DT_F32)
        checksum_kernel<DT_F32><<<g, 256, 0, s>>>(buf, count, aligned,
                                                   reinterpret_cast<unsigned long long *>(hash));
    else
        checksum_kernel<DT_BF16><<<g, 256, 0, s>>>(buf, count, aligned,
                                                    reinterpret_cast<unsigned long long *>(hash));
    return hipGetLastError();
}

hipError_t launch_checksum_sum(const void *buf, int64_t count, int dt, uint64_t *hash, double *sum,
                               double *part, int64_t cap, hipStream_t s)
{
    if (hash) {
        fill_u32_kernel<<<1, 64, 0, s>>>(reinterpret_cast<uint32_t *>(hash), 2, 0u);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    const int64_t T = ceil_div(count, SUM_TILE);
    if (T > 0) {
        const bool aligned = (reinterpret_cast<uintptr_t>(buf) & 15u) == 0;
        const unsigned g = grid_for(T, 1, cap);
        auto *hp = reinterpret_cast<unsigned long long *>(hash);
        if (dt == DT_F32) {
            if (hash)
                checksum_sum_kernel<DT_F32, true><<<g, 256, 0, s>>>(buf, count, aligned, hp, part);
            else
                checksum_sum_kernel<DT_F32, false><<<g, 256, 0, s>>>(buf, count, aligned, hp, part);
        } else {
            if (hash)
                checksum_sum_kernel<DT_BF16, true><<<g, 256, 0, s>>>(buf, count, aligned, hp, part);
            else
                checksum_sum_kernel<DT_BF16, false><<<g, 256, 0, s>>>(buf, count, aligned, hp, part);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    sum_finish_kernel<<<1, SUM_FINISH_THREADS, 0, s>>>(part, T, sum);
    return hipGetLastError();
}

hipError_t launch_fill_u32(void *p, int64_t words, uint32_t value, hipStream_t s)
{
    if (words <= 0)
        return hipSuccess;
    fill_u32_kernel<<<grid_for(words, 256, 8192), 256, 0, s>>>(static_cast<uint32_t *>(p), words, value);
    return hipGetLastError();
}

hipError_t launch_fill_bytes(void *p, int64_t bytes, uint8_t value, hipStream_t s)
{
    // whole words from a 4-byte aligned start, then the last 0-3 bytes alone,
    // so nothing past p[bytes-1] is written
    if (bytes <= 0)
        return hipSuccess;
    const uint32_t v4 = value * 0x01010101u;
    hipError_t e = launch_fill_u32(p, bytes / 4, v4, s);
    if (e == hipSuccess && (bytes & 3) != 0) {
        fill_u8_kernel<<<1, 64, 0, s>>>(static_cast<uint8_t *>(p) + (bytes & ~int64_t(3)), bytes & 3,
                                        value);
        e = hipGetLastError();
    }
    return e;
}

hipError_t launch_convert(const void *src, int sdt, void *dst, int ddt, int64_t N, hipStream_t s)
{
    if (N <= 0)
        return hipSuccess;
    const unsigned g = grid_for(N, 256, 65536);
    if (sdt == DT_F32 && ddt == DT_F32)
        convert_kernel<DT_F32, DT_F32><<<g, 256, 0, s>>>(src, dst, N);
    else if (sdt == DT_F32)
        convert_kernel<DT_F32, DT_BF16><<<g, 256, 0, s>>>(src, dst, N);
    else if (ddt == DT_F32)
        convert_kernel<DT_BF16, DT_F32><<<g, 256, 0, s>>>(src, dst, N);
    else
        convert_kernel<DT_BF16, DT_BF16><<<g, 256, 0, s>>>(src, dst, N);
    return hipGetLastError();
}

} // namespace fa
