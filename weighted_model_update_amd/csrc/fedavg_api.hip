// Host side of the FedAvg aggregation library: the extern "C" entry points of
// include/fedavg.h -- argument checks, weight sums in exact integers, launch
// shapes, and the streaming pipeline (staging slots, copy/compute streams,
// events, per-client coverage).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <unordered_map>
#include <vector>

#include "fedavg_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok()
{
    g_last_error.clear();
    return FA_OK;
}

int hip_fail(hipError_t e, const char *what)
{
    return fail(FA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool dtype_ok(int d) { return d == FA_F32 || d == FA_BF16; }
size_t dsize(int d) { return d == FA_F32 ? 4 : 2; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Two byte ranges either coincide exactly or do not overlap at all.
bool overlap_ok(const void *a, size_t abytes, const void *b, size_t bbytes)
{
    if (!a || !b || abytes == 0 || bbytes == 0)
        return true;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    if (a0 == b0 && abytes == bbytes)
        return true;
    return a0 + abytes <= b0 || b0 + bbytes <= a0;
}

// Launch-shape options (fedavg_set_option).
int64_t g_blocks_per_cu = 0;     // grid-stride cap, workgroups per CU (0: none)
int64_t g_resident_per_cu = -1;  // dense kernel: resident workgroups per CU (0: no cap,
                                 // -1: by client count, dense_resident_for)
int64_t g_mask_vpb = 2048;       // masked kernel: 8-parameter vectors per block
int64_t g_sparse_blocks = 0;     // sparse merge: parameter ranges (0: the default rule)
int64_t g_sparse_tile = fa::SP_DEFAULT_TILE;
int64_t g_index_tiles = 0;       // client-at-a-time sparse: 0 by density, 1 scatter, 2 tiles
// Resident workgroups per CU of the streaming kernels (by residency_lds).
// Measured on MI355X over 2^31 parameters held in HBM, as fractions of HBM
// peak, caps 0 (none), 1, 2, 3, 4, 6: the accumulate (a bf16 chunk into the
// fp32 sums) 0.73, 0.51, 0.78, 0.82, 0.79, 0.75; the two-level merge (an
// fp32 partial into the sums) 0.77, 0.61, 0.81, 0.80, 0.79, 0.76; the
// finalize to bf16 0.79, 0.42, 0.65, 0.76, 0.81, 0.79.
constexpr int STREAM_ACC_RESIDENT = 3;
constexpr int STREAM_MERGE_RESIDENT = 2;
constexpr int STREAM_FIN_RESIDENT = 4;
constexpr int64_t SPARSE_MAX_BLOCKS = 1 << 19;
constexpr int64_t SPARSE_RANGE_TILES = 4;  // default: tiles per range
constexpr int64_t SPARSE_MIN_RANGES = 4096; // default: ranges while there are that many tiles
constexpr int64_t SPARSE_MIN_TILE = 512;
constexpr size_t HEADER_BYTES = 256;
constexpr int64_t INDEX_TILES_MIN_LEN = 1 << 16; // shorter lists are scattered

int cu_count()
{
    // per device, filled on first use; threads that race store the same value
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

int64_t grid_cap() { return g_blocks_per_cu > 0 ? g_blocks_per_cu * cu_count() : 0; }

// Resident dense workgroups per CU when the caller sets none.  A lane keeps
// one 16-byte load per client in flight, so the bytes a CU has in flight
// grow with K; past a point more of them only queue.  Measured on MI355X
// at 65.3 GB per launch (bf16 clients and output), two allocations on two
// devices, best cap per client count (fraction of HBM peak there):
//   K = 2: none (0.78)   K = 3: 4 or 6 (0.77)   K = 4, 5: 4 (0.77-0.80, 0.75)
//   K = 6, 7, 8, 10: 3 (0.73-0.75)   K = 12, 14: none (0.71-0.76)
//   K = 16: 2 (0.74-0.75; 0.73 at 3)   K = 20 ... 64: none (0.72-0.74)
int dense_resident_for(int K)
{
    if (K <= 2)
        return 0;
    if (K <= 5)
        return 4;
    if (K <= 10)
        return 3;
    if (K < 16)
        return 0;
    return K == 16 ? 2 : 0;
}

enum class Residence { Device, PinnedHost, Pageable };

Residence residence_of(const void *p)
{
    hipPointerAttribute_t attr;
    std::memset(&attr, 0, sizeof attr);
    hipError_t e = hipPointerGetAttributes(&attr, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return Residence::Pageable;
    }
    if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged)
        return Residence::Device;
    if (attr.type == hipMemoryTypeHost)
        return Residence::PinnedHost;
    return Residence::Pageable;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

size_t slot_bytes(int64_t chunk_bytes, int partial)
{
    // values, plus room for a mask or an index list of the largest chunk
    // (at most chunk_bytes/2 entries, 8 bytes each)
    size_t b = round_up((size_t)chunk_bytes, 256);
    if (partial)
        b += round_up((size_t)chunk_bytes * 4, 256);
    return b;
}

// ------------------------------------------------------------ spill / resume
//
// Exported state (host bytes, little-endian):
//   u32 magic "FAST", u32 version, i64 N, i32 mode, i32 partial, i32 has_count,
//   i32 finalized, u32 clients, u32 reserved, then per client
//   {i32 id, i32 members, i64 weight, i64 covered}, then u64 FNV-1a of all the
//   bytes before it.

constexpr uint32_t STATE_MAGIC = 0x54534146u; // "FAST"
constexpr uint32_t STATE_VERSION = 1;
constexpr size_t STATE_HEAD = 4 + 4 + 8 + 4 * 4 + 4 + 4;
constexpr size_t STATE_CLIENT = 4 + 4 + 8 + 8;

uint64_t fnv1a64(const unsigned char *p, size_t n)
{
    uint64_t h = 0xcbf29ce484222325ull;
    for (size_t i = 0; i < n; ++i) {
        h ^= p[i];
        h *= 0x100000001b3ull;
    }
    return h;
}

template <class T> void put(unsigned char *&p, T v)
{
    std::memcpy(p, &v, sizeof v);
    p += sizeof v;
}

template <class T> T get(const unsigned char *&p)
{
    T v;
    std::memcpy(&v, p, sizeof v);
    p += sizeof v;
    return v;
}

} // namespace

// ============================================================ streaming state

struct fa_stream_state {
    struct Client {
        int64_t n;       // weight: n_k, or a merged partial's W
        int64_t covered; // dense: next expected offset; partial: end of the last range
        int members;     // clients behind it: 1, or a merged partial's client count
    };
    int device = 0;
    int64_t N = 0;
    int mode = FA_WEIGHTS;
    int partial = 0;
    float *acc = nullptr;
    uint32_t *wsum = nullptr;
    uint8_t *count = nullptr;
    char *staging = nullptr;
    int64_t chunk_bytes = 0;
    size_t slot_size = 0;
    int n_slots = 0;
    hipStream_t compute = nullptr;
    hipStream_t copy = nullptr;
    bool own_copy = false;
    // copy_done[j]: the host-to-device copy of the call whose number is j
    // modulo n_slots (recorded only when that call staged); slot_free[s]: the
    // last kernel that read staging slot s
    std::vector<hipEvent_t> copy_done, slot_free;
    std::vector<bool> copy_pending, slot_used;
    int64_t calls = 0;  // accumulate calls of any kind on this handle
    int64_t staged = 0; // calls that staged host memory (slot round robin)
    int ring = 0;       // copy_done entry of the current call
    bool finalized = false;
    std::unordered_map<int, Client> clients;
    int *err_flag() { return reinterpret_cast<int *>(staging); }
    // the tiled index path's verdict on a list (its own 128-byte line)
    int *list_gate() { return reinterpret_cast<int *>(staging + 128); }
    uint64_t total_weight() const
    {
        uint64_t S = 0;
        for (auto &c : clients)
            S += (uint64_t)c.second.n;
        return S;
    }
    int64_t total_members() const
    {
        int64_t m = 0;
        for (auto &c : clients)
            m += c.second.members;
        return m;
    }
    // Admits a new client (or merged partial) of weight n standing for
    // `members` clients; returns an error status, or FA_OK.
    int admit(int64_t n, int members)
    {
        if (partial && total_members() + members > FA_MAX_STREAM_CLIENTS)
            return fail(FA_ERR_RANGE, "more than %d clients in partial mode", FA_MAX_STREAM_CLIENTS);
        if (total_weight() + (uint64_t)n >= (1ull << 32))
            return fail(FA_ERR_RANGE, "sum of weights must be below 2^32");
        return FA_OK;
    }
    // Checks a chunk's range against the client's coverage and advances it.
    int cover(int client_id, Client &cl, int64_t offset, int64_t len)
    {
        if (!partial) {
            if (offset != cl.covered)
                return fail(FA_ERR_ARG,
                            "dense mode: client %d chunk starts at %lld, expected %lld (chunks "
                            "must arrive in order and tile [0,N))",
                            client_id, (long long)offset, (long long)cl.covered);
        } else if (offset < cl.covered) {
            return fail(FA_ERR_ARG, "client %d ranges must be ascending and non-overlapping",
                        client_id);
        }
        cl.covered = offset + len;
        return FA_OK;
    }
    // Opens an accumulate call.  A host buffer handed to call j may be reused
    // once n_slots further calls have returned: call j + n_slots waits here
    // for call j's copy, whatever kinds of calls came in between (device
    // chunks, empty chunks, zero weights and refused calls count too).
    // Returns FA_OK or the failure of the wait.
    int open_call()
    {
        ring = (int)(calls % n_slots);
        ++calls;
        if (copy_pending[ring]) {
            const hipError_t e = hipEventSynchronize(copy_done[ring]);
            if (e != hipSuccess)
                return hip_fail(e, "waiting for an earlier copy");
            copy_pending[ring] = false;
        }
        return FA_OK;
    }
    // Stages `parts` host arrays into the next slot (host buffers given as
    // (src, bytes, offset in slot)); returns the slot, or -1 after a failure
    // of a HIP call (recorded as FA_ERR_HIP).
    int stage(const void *const *src, const size_t *bytes, const size_t *at, int parts)
    {
        const int sl = (int)(staged % n_slots);
        hipError_t e = hipSuccess;
        // the slot is free once the kernel that last read it is done
        if (slot_used[sl])
            e = hipStreamWaitEvent(copy, slot_free[sl], 0);
        for (int i = 0; i < parts && e == hipSuccess; ++i)
            if (src[i] && bytes[i])
                e = hipMemcpyAsync(slot(sl) + at[i], src[i], bytes[i], hipMemcpyHostToDevice, copy);
        if (e == hipSuccess)
            e = hipEventRecord(copy_done[ring], copy);
        if (e == hipSuccess)
            copy_pending[ring] = true;
        if (e == hipSuccess)
            e = hipStreamWaitEvent(compute, copy_done[ring], 0);
        if (e != hipSuccess) {
            hip_fail(e, "staging copy");
            return -1;
        }
        return sl;
    }
    // Marks a staged slot busy until the kernel just launched on it is done.
    int release(int sl)
    {
        hipError_t e = hipEventRecord(slot_free[sl], compute);
        if (e != hipSuccess)
            return hip_fail(e, "event record");
        slot_used[sl] = true;
        ++staged;
        return FA_OK;
    }
    char *slot(int s) { return staging + HEADER_BYTES + (size_t)s * slot_size; }
};

extern "C" {

int fedavg_abi_version(void) { return FEDAVG_ABI_VERSION; }

int fedavg_arena_layout(int count, int64_t bytes, int64_t *offsets, int64_t *total_bytes)
{
    if (count < 1 || count > FA_ARENA_MAX_BUFFERS)
        return fail(FA_ERR_ARG, "count=%d outside [1, %d]", count, FA_ARENA_MAX_BUFFERS);
    if (bytes < 0 || !offsets || !total_bytes)
        return fail(FA_ERR_ARG, "need bytes >= 0 and both result pointers");
    constexpr int64_t PAGE = (int64_t)2 << 20, STAGGER = (int64_t)32 << 10, LIMIT = (int64_t)1 << 62;
    if (bytes > LIMIT - PAGE)
        return fail(FA_ERR_RANGE, "bytes=%lld is too large", (long long)bytes);
    // each buffer rounded up to whole pages, then one stagger step more
    const int64_t pitch = (bytes + PAGE - 1) / PAGE * PAGE + STAGGER;
    if ((int64_t)(count - 1) > (LIMIT - bytes) / pitch)
        return fail(FA_ERR_RANGE, "%d buffers of %lld bytes exceed 2^62 bytes", count, (long long)bytes);
    for (int j = 0; j < count; ++j)
        offsets[j] = (int64_t)j * pitch;
    *total_bytes = (int64_t)(count - 1) * pitch + bytes;
    return ok();
}

const char *fedavg_last_error(void) { return g_last_error.c_str(); }

int fedavg_set_option(int option, int64_t value)
{
    switch (option) {
    case FA_OPT_BLOCKS_PER_CU:
        if (value < 0 || value > 1024)
            return fail(FA_ERR_RANGE, "blocks per CU must be in [0, 1024]");
        g_blocks_per_cu = value;
        return ok();
    case FA_OPT_MASK_VECTORS_PER_BLOCK:
        if (value < 1 || value > (1 << 24))
            return fail(FA_ERR_RANGE, "vectors per block must be in [1, 2^24]");
        g_mask_vpb = value;
        return ok();
    case FA_OPT_RESIDENT_PER_CU:
        if (value < -1 || value > 32)
            return fail(FA_ERR_RANGE, "resident workgroups per CU must be in [-1, 32]");
        g_resident_per_cu = value;
        return ok();
    case FA_OPT_SPARSE_TILE:
        if (value != 512 && value != 1024 && value != 2048 && value != 4096 && value != 8192)
            return fail(FA_ERR_RANGE, "sparse tile must be 512, 1024, 2048, 4096 or 8192");
        g_sparse_tile = value;
        return ok();
    case FA_OPT_TOPK_SAMPLED:
        if (value != 0 && value != 1)
            return fail(FA_ERR_RANGE, "top-k sampled path must be 0 or 1");
        fa::topk_set_sampled((int)value);
        return ok();
    case FA_OPT_INDEX_TILES:
        if (value < 0 || value > 2)
            return fail(FA_ERR_RANGE, "index tiles must be 0, 1 or 2");
        g_index_tiles = value;
        return ok();
    case FA_OPT_SPARSE_BLOCKS:
        if (value < 0 || value > SPARSE_MAX_BLOCKS)
            return fail(FA_ERR_RANGE, "sparse blocks must be in [0, %lld]",
                        (long long)SPARSE_MAX_BLOCKS);
        g_sparse_blocks = value;
        return ok();
    default:
        return fail(FA_ERR_ARG, "unknown option %d", option);
    }
}

// ============================================================ resident

int fedavg_aggregate(int K, const void *const *x, fa_dtype x_dtype, const int64_t *n, int64_t N,
                     fa_mode mode, const void *base, fa_dtype base_dtype, void *out,
                     fa_dtype out_dtype, int T, const int64_t *seg_bounds, const uint8_t *present,
                     void *stream)
{
    if (K < 1 || K > FA_MAX_CLIENTS)
        return fail(FA_ERR_RANGE, "K=%d outside [1, %d]", K, FA_MAX_CLIENTS);
    if (!x || !n)
        return fail(FA_ERR_ARG, "x and n must not be NULL");
    if (N < 0)
        return fail(FA_ERR_ARG, "N=%lld is negative", (long long)N);
    if (N > FA_MAX_N)
        return fail(FA_ERR_RANGE, "N=%lld exceeds 2^40", (long long)N);
    if (!dtype_ok(x_dtype) || !dtype_ok(out_dtype) || !dtype_ok(base_dtype))
        return fail(FA_ERR_DTYPE, "dtypes must be FA_F32 or FA_BF16");
    if (mode != FA_WEIGHTS && mode != FA_DELTAS && mode != FA_DELTAS_ZERO_FILL)
        return fail(FA_ERR_ARG, "unknown mode %d", (int)mode);
    if (T < 0)
        return fail(FA_ERR_ARG, "T=%d is negative", T);
    // an empty model is a no-op: its (empty) buffers may be NULL
    if (N > 0 && mode != FA_WEIGHTS && !base)
        return fail(FA_ERR_ARG, "delta modes need base");
    // kernels see weights or deltas; zero fill only changes the divisor of
    // the masked path (with every client sending everything, W_i = S)
    const int kmode = mode == FA_WEIGHTS ? FA_WEIGHTS : FA_DELTAS;
    if (N > 0 && T > 0 && (!base || !seg_bounds || !present))
        return fail(FA_ERR_ARG, "segment masks need base, seg_bounds and present");
    if (N > 0 && !out)
        return fail(FA_ERR_ARG, "out must not be NULL");

    fa::DenseArgs d;
    std::memset(&d, 0, sizeof d);
    fa::MaskedArgs m;
    std::memset(&m, 0, sizeof m);
    int Kc = 0;
    uint64_t S = 0;
    const size_t xbytes = (size_t)N * dsize(x_dtype), obytes = (size_t)N * dsize(out_dtype);
    bool aligned = aligned16(out);
    for (int k = 0; k < K; ++k) {
        if (n[k] < 0 || n[k] > FA_MAX_WEIGHT)
            return fail(FA_ERR_RANGE, "n[%d]=%lld outside [0, 2^24]", k, (long long)n[k]);
        if (n[k] == 0)
            continue;
        if (!x[k] && N > 0)
            return fail(FA_ERR_ARG, "x[%d] is NULL", k);
        if (!overlap_ok(out, obytes, x[k], xbytes))
            return fail(FA_ERR_ARG, "out partially overlaps x[%d]", k);
        aligned = aligned && aligned16(x[k]);
        d.x[Kc] = m.x[Kc] = x[k];
        d.w[Kc] = m.w[Kc] = (float)n[k];
        m.wi[Kc] = (uint32_t)n[k];
        m.row[Kc] = k;
        S += (uint64_t)n[k];
        ++Kc;
    }
    if (S >= (1ull << 32))
        return fail(FA_ERR_RANGE, "sum of n_k must be below 2^32");
    // the dense kernel's last batch of clients adds its unused slots with
    // weight -0, which changes no accumulator bit
    for (int k = Kc; k < FA_MAX_CLIENTS; ++k)
        d.w[k] = -0.0f;
    if (base && !overlap_ok(out, obytes, base, (size_t)N * dsize(base_dtype)))
        return fail(FA_ERR_ARG, "out partially overlaps base");
    if (N == 0)
        return ok();
    hipStream_t s = static_cast<hipStream_t>(stream);

    if (T == 0) {
        if (S == 0) {
            if (mode == FA_WEIGHTS)
                return fail(FA_ERR_ZERO_WEIGHT, "sum of n_k is 0 in dense weights mode");
            // no contributor: every parameter keeps the global value
            hipError_t e = fa::launch_convert(base, base_dtype, out, out_dtype, N, s);
            return e == hipSuccess ? ok() : hip_fail(e, "convert launch");
        }
        if (kmode == FA_DELTAS)
            aligned = aligned && aligned16(base);
        d.K = Kc;
        d.N = N;
        d.base = base;
        d.out = out;
        d.S = (float)S;
        const int resident = g_resident_per_cu >= 0 ? (int)g_resident_per_cu : dense_resident_for(Kc);
        hipError_t e = fa::launch_dense(d, x_dtype, out_dtype, base_dtype, kmode, aligned,
                                        grid_cap(), resident, s);
        return e == hipSuccess ? ok() : hip_fail(e, "dense aggregate launch");
    }

    aligned = aligned && aligned16(base);
    m.K = Kc;
    m.T = T;
    m.N = N;
    m.vpb = g_mask_vpb;
    m.bounds = seg_bounds;
    m.present = present;
    m.base = base;
    m.out = out;
    m.zero_fill = mode == FA_DELTAS_ZERO_FILL;
    m.S_all = (float)S;
    hipError_t e = fa::launch_masked(m, x_dtype, out_dtype, base_dtype, kmode, aligned, s);
    return e == hipSuccess ? ok() : hip_fail(e, "masked aggregate launch");
}

// ============================================================ streaming

int fedavg_workspace_size(int64_t N, int partial, int64_t chunk_bytes, int n_slots,
                          size_t *acc_bytes, size_t *wsum_bytes, size_t *count_bytes,
                          size_t *staging_bytes)
{
    if (N < 0 || chunk_bytes <= 0 || n_slots < 1)
        return fail(FA_ERR_ARG, "need N >= 0, chunk_bytes > 0, n_slots >= 1");
    if (N > FA_MAX_N || chunk_bytes > FA_MAX_N || n_slots > 64)
        return fail(FA_ERR_RANGE, "need N <= 2^40, chunk_bytes <= 2^40, n_slots <= 64");
    if (partial != 0 && partial != 1)
        return fail(FA_ERR_ARG, "partial must be 0 or 1");
    if (acc_bytes)
        *acc_bytes = (size_t)N * 4;
    if (wsum_bytes)
        *wsum_bytes = partial ? (size_t)N * 4 : 0;
    if (count_bytes)
        *count_bytes = partial ? (size_t)N : 0;
    if (staging_bytes)
        *staging_bytes = HEADER_BYTES + (size_t)n_slots * slot_bytes(chunk_bytes, partial);
    return ok();
}

// Checks begin/resume arguments and creates the handle with its events and
// copy stream; device buffers are not touched.
static int open_handle(fa_handle *h, int64_t N, int mode, int partial, float *acc, uint32_t *wsum,
                       uint8_t *count, void *staging, size_t staging_bytes, int64_t chunk_bytes,
                       int n_slots, void *compute_stream, void *copy_stream)
{
    if (!h)
        return fail(FA_ERR_ARG, "handle pointer is NULL");
    *h = nullptr;
    if (N < 0 || chunk_bytes <= 0 || n_slots < 1)
        return fail(FA_ERR_ARG, "need N >= 0, chunk_bytes > 0, n_slots >= 1");
    if (N > FA_MAX_N || chunk_bytes > FA_MAX_N || n_slots > 64)
        return fail(FA_ERR_RANGE, "need N <= 2^40, chunk_bytes <= 2^40, n_slots <= 64");
    if (mode != FA_WEIGHTS && mode != FA_DELTAS && mode != FA_DELTAS_ZERO_FILL)
        return fail(FA_ERR_ARG, "unknown mode %d", mode);
    if (partial != 0 && partial != 1)
        return fail(FA_ERR_ARG, "partial must be 0 or 1");
    if (!acc || !staging || (partial && !wsum))
        return fail(FA_ERR_WORKSPACE, "acc, staging (and wsum in partial mode) are required");
    size_t need = HEADER_BYTES + (size_t)n_slots * slot_bytes(chunk_bytes, partial);
    if (staging_bytes < need)
        return fail(FA_ERR_WORKSPACE, "staging has %zu bytes, needs %zu", staging_bytes, need);
    if (!aligned16(acc) || !aligned16(staging) || (wsum && !aligned16(wsum)) ||
        (count && !aligned16(count)))
        return fail(FA_ERR_ARG, "acc, wsum, count and staging must be 16-byte aligned");

    fa_stream_state *st = new (std::nothrow) fa_stream_state();
    if (!st)
        return fail(FA_ERR_ARG, "out of host memory");
    (void)hipGetDevice(&st->device);
    st->N = N;
    st->mode = mode;
    st->partial = partial;
    st->acc = acc;
    st->wsum = partial ? wsum : nullptr;
    st->count = partial ? count : nullptr;
    st->staging = static_cast<char *>(staging);
    st->chunk_bytes = chunk_bytes;
    st->slot_size = slot_bytes(chunk_bytes, partial);
    st->n_slots = n_slots;
    st->compute = static_cast<hipStream_t>(compute_stream);
    st->copy = static_cast<hipStream_t>(copy_stream);
    hipError_t e = hipSuccess;
    if (!st->copy) {
        e = hipStreamCreateWithFlags(&st->copy, hipStreamNonBlocking);
        if (e != hipSuccess) {
            delete st;
            return hip_fail(e, "copy stream");
        }
        st->own_copy = true;
    }
    st->copy_done.resize(n_slots);
    st->slot_free.resize(n_slots);
    st->copy_pending.assign(n_slots, false);
    st->slot_used.assign(n_slots, false);
    for (int i = 0; i < n_slots && e == hipSuccess; ++i) {
        e = hipEventCreateWithFlags(&st->copy_done[i], hipEventDisableTiming);
        if (e == hipSuccess)
            e = hipEventCreateWithFlags(&st->slot_free[i], hipEventDisableTiming);
    }
    // the staging header holds the deferred error flag
    if (e == hipSuccess)
        e = fa::launch_fill_u32(st->staging, HEADER_BYTES / 4, 0u, st->compute);
    // The caller's buffers are ordered by compute_stream, but the copies into
    // the staging slots run on the copy stream: work already queued on the
    // compute stream may still write that memory (a caching allocator hands
    // out memory whose previous owner's kernels are still running on that
    // stream).  Every slot counts as busy until the compute stream reaches
    // this point, so the first copy into each slot waits for it.
    for (int i = 0; i < n_slots && e == hipSuccess; ++i) {
        e = hipEventRecord(st->slot_free[i], st->compute);
        st->slot_used[i] = true;
    }
    if (e != hipSuccess) {
        fedavg_destroy(st);
        return hip_fail(e, "handle set-up");
    }
    *h = st;
    return FA_OK;
}

int fedavg_begin(fa_handle *h, int64_t N, fa_mode mode, int partial, float *acc, uint32_t *wsum,
                 uint8_t *count, void *staging, size_t staging_bytes, int64_t chunk_bytes,
                 int n_slots, void *compute_stream, void *copy_stream)
{
    int rc = open_handle(h, N, mode, partial, acc, wsum, count, staging, staging_bytes, chunk_bytes,
                         n_slots, compute_stream, copy_stream);
    if (rc != FA_OK)
        return rc;
    fa_stream_state *st = *h;
    hipError_t e = fa::launch_fill_u32(acc, N, 0u, st->compute);
    if (e == hipSuccess && st->partial)
        e = fa::launch_fill_u32(st->wsum, N, 0u, st->compute);
    if (e == hipSuccess && st->count)
        e = fa::launch_fill_bytes(st->count, N, 0, st->compute);
    if (e != hipSuccess) {
        fedavg_destroy(st);
        *h = nullptr;
        return hip_fail(e, "begin");
    }
    return ok();
}

int fedavg_state_size(fa_handle h, size_t *bytes)
{
    if (!h || !bytes)
        return fail(FA_ERR_ARG, "need a handle and a result pointer");
    *bytes = STATE_HEAD + h->clients.size() * STATE_CLIENT + 8;
    return ok();
}

int fedavg_export_state(fa_handle h, void *buf, size_t bytes)
{
    if (!h || !buf)
        return fail(FA_ERR_ARG, "need a handle and a buffer");
    fa_stream_state &st = *h;
    const size_t need = STATE_HEAD + st.clients.size() * STATE_CLIENT + 8;
    if (bytes < need)
        return fail(FA_ERR_ARG, "state buffer has %zu bytes, needs %zu", bytes, need);
    // the accumulator must be final before the caller copies it out
    int rc = fedavg_sync(h);
    if (rc != FA_OK)
        return rc;
    std::vector<std::pair<int, fa_stream_state::Client>> cl(st.clients.begin(), st.clients.end());
    std::sort(cl.begin(), cl.end(), [](const auto &a, const auto &b) { return a.first < b.first; });
    unsigned char *p = static_cast<unsigned char *>(buf);
    unsigned char *p0 = p;
    put<uint32_t>(p, STATE_MAGIC);
    put<uint32_t>(p, STATE_VERSION);
    put<int64_t>(p, st.N);
    put<int32_t>(p, st.mode);
    put<int32_t>(p, st.partial);
    put<int32_t>(p, st.count ? 1 : 0);
    put<int32_t>(p, st.finalized ? 1 : 0);
    put<uint32_t>(p, (uint32_t)cl.size());
    put<uint32_t>(p, 0u);
    for (auto &c : cl) {
        put<int32_t>(p, c.first);
        put<int32_t>(p, c.second.members);
        put<int64_t>(p, c.second.n);
        put<int64_t>(p, c.second.covered);
    }
    put<uint64_t>(p, fnv1a64(p0, (size_t)(p - p0)));
    return ok();
}

int fedavg_resume(fa_handle *h, const void *state, size_t state_bytes, int64_t N_expect,
                  fa_mode mode_expect, int partial_expect, float *acc, uint32_t *wsum,
                  uint8_t *count, void *staging, size_t staging_bytes, int64_t chunk_bytes,
                  int n_slots, void *compute_stream, void *copy_stream)
{
    if (h)
        *h = nullptr;
    if (!state || state_bytes < STATE_HEAD + 8)
        return fail(FA_ERR_ARG, "state is missing or too short");
    const unsigned char *p = static_cast<const unsigned char *>(state);
    const unsigned char *p0 = p;
    if (get<uint32_t>(p) != STATE_MAGIC)
        return fail(FA_ERR_ARG, "not an exported accumulator state");
    if (get<uint32_t>(p) != STATE_VERSION)
        return fail(FA_ERR_ARG, "unsupported state version");
    const int64_t N = get<int64_t>(p);
    const int32_t mode = get<int32_t>(p);
    const int32_t partial = get<int32_t>(p);
    const int32_t has_count = get<int32_t>(p);
    const int32_t finalized = get<int32_t>(p);
    const uint32_t nc = get<uint32_t>(p);
    (void)get<uint32_t>(p);
    if (nc > (1u << 20) || state_bytes != STATE_HEAD + (size_t)nc * STATE_CLIENT + 8)
        return fail(FA_ERR_ARG, "state size does not match its client count");
    {
        const unsigned char *q = p0 + STATE_HEAD + (size_t)nc * STATE_CLIENT;
        if (get<uint64_t>(q) != fnv1a64(p0, STATE_HEAD + (size_t)nc * STATE_CLIENT))
            return fail(FA_ERR_ARG, "state checksum mismatch");
    }
    if (N < 0 || (partial != 0 && partial != 1) || (has_count != 0 && has_count != 1) ||
        (finalized != 0 && finalized != 1) || (!partial && has_count))
        return fail(FA_ERR_ARG, "state header is inconsistent");
    if (N != N_expect || mode != (int32_t)mode_expect || partial != partial_expect)
        return fail(FA_ERR_ARG, "state is for N=%lld mode=%d partial=%d, not N=%lld mode=%d partial=%d",
                    (long long)N, mode, partial, (long long)N_expect, (int)mode_expect,
                    partial_expect);
    if ((bool)has_count != (partial && count != nullptr))
        return fail(FA_ERR_ARG, "the state %s client counts; pass a count buffer %s",
                    has_count ? "has" : "has no", has_count ? "(restored)" : "of NULL");
    std::unordered_map<int, fa_stream_state::Client> clients;
    uint64_t S = 0;
    int64_t members = 0;
    for (uint32_t i = 0; i < nc; ++i) {
        const int32_t id = get<int32_t>(p);
        fa_stream_state::Client c;
        c.members = get<int32_t>(p);
        c.n = get<int64_t>(p);
        c.covered = get<int64_t>(p);
        if (id < 0 || clients.count(id) || c.members < 1 || c.n <= 0 || c.n >= (1ll << 32) ||
            c.covered < 0 || c.covered > N)
            return fail(FA_ERR_ARG, "state client record %u is invalid", i);
        S += (uint64_t)c.n;
        members += c.members;
        clients[id] = c;
    }
    if (S >= (1ull << 32) || (partial && members > FA_MAX_STREAM_CLIENTS))
        return fail(FA_ERR_ARG, "state totals exceed the handle limits");

    int rc = open_handle(h, N, mode, partial, acc, wsum, count, staging, staging_bytes, chunk_bytes,
                         n_slots, compute_stream, copy_stream);
    if (rc != FA_OK)
        return rc;
    (*h)->clients = std::move(clients);
    (*h)->finalized = finalized != 0;
    return ok();
}

int fedavg_accumulate(fa_handle h, int client_id, int64_t n_k, const void *chunk, fa_dtype dtype,
                      int64_t offset, int64_t len, const uint8_t *mask, const int64_t *indices)
{
    if (!h)
        return fail(FA_ERR_ARG, "NULL handle");
    fa_stream_state &st = *h;
    {
        const int rc = st.open_call();
        if (rc != FA_OK)
            return rc;
    }
    if (st.finalized)
        return fail(FA_ERR_STATE, "accumulate after finalize");
    if (client_id < 0)
        return fail(FA_ERR_ARG, "client_id must be >= 0");
    if (n_k < 0 || n_k > FA_MAX_WEIGHT)
        return fail(FA_ERR_RANGE, "n_k=%lld outside [0, 2^24]", (long long)n_k);
    if (!dtype_ok(dtype))
        return fail(FA_ERR_DTYPE, "chunk dtype must be FA_F32 or FA_BF16");
    if (len < 0 || offset < 0)
        return fail(FA_ERR_ARG, "offset and len must be >= 0");
    if (mask && indices)
        return fail(FA_ERR_ARG, "pass a mask or indices, not both");
    if ((mask || indices) && !st.partial)
        return fail(FA_ERR_ARG, "masks and indices need a partial-mode handle");
    // written so that no sum can overflow: offset + len may exceed 2^63
    if (!indices && (offset > st.N || len > st.N - offset))
        return fail(FA_ERR_RANGE, "chunk at %lld of %lld elements exceeds N=%lld", (long long)offset,
                    (long long)len, (long long)st.N);
    if (indices && offset > st.N)
        return fail(FA_ERR_RANGE, "offset beyond N");
    if (len > 0 && !chunk)
        return fail(FA_ERR_ARG, "chunk is NULL");

    auto it = st.clients.find(client_id);
    if (it != st.clients.end() && (it->second.n != n_k || it->second.members != 1))
        return fail(FA_ERR_ARG, "client %d changed its n_k", client_id);
    if (n_k == 0)
        return ok();
    if (it == st.clients.end()) {
        const int rc = st.admit(n_k, 1);
        if (rc != FA_OK)
            return rc;
    }
    fa_stream_state::Client cl =
        it != st.clients.end() ? it->second : fa_stream_state::Client{n_k, 0, 1};
    // an empty chunk carries no parameter: it enters the client (and counts
    // as a call) but is outside the ordering and tiling rules
    if (len == 0) {
        st.clients[client_id] = cl;
        return ok();
    }
    if (!indices) {
        const int rc = st.cover(client_id, cl, offset, len);
        if (rc != FA_OK)
            return rc;
    }

    const size_t esize = dsize(dtype);
    const size_t vbytes = (size_t)len * esize;
    const Residence res = residence_of(chunk);
    if (res == Residence::Pageable)
        return fail(FA_ERR_ARG, "chunk must be pinned host memory or device memory");
    if (mask && residence_of(mask) != res)
        return fail(FA_ERR_ARG, "mask must live where the chunk lives");
    if (indices && residence_of(indices) != res)
        return fail(FA_ERR_ARG, "indices must live where the chunk lives");

    fa::StreamArgs a;
    std::memset(&a, 0, sizeof a);
    a.acc = st.acc;
    a.wsum = st.wsum;
    a.count = st.count;
    a.offset = offset;
    a.len = len;
    a.N = st.N;
    a.w = (float)n_k;
    a.wi = (uint32_t)n_k;
    a.err = st.err_flag();

    hipError_t e = hipSuccess;
    int slot = -1;
    if (res == Residence::PinnedHost) {
        if (vbytes > (size_t)st.chunk_bytes)
            return fail(FA_ERR_RANGE, "chunk of %zu bytes exceeds chunk_bytes=%lld", vbytes,
                        (long long)st.chunk_bytes);
        const size_t aux_at = round_up((size_t)st.chunk_bytes, 256);
        const void *src[2] = {chunk, mask ? (const void *)mask : (const void *)indices};
        const size_t bytes[2] = {vbytes, mask ? (size_t)len : (indices ? (size_t)len * 8 : 0)};
        const size_t at[2] = {0, aux_at};
        slot = st.stage(src, bytes, at, 2);
        if (slot < 0)
            return FA_ERR_HIP; // message recorded by stage()
        char *dst = st.slot(slot);
        char *aux = dst + aux_at;
        a.chunk = dst;
        a.mask = mask ? reinterpret_cast<const uint8_t *>(aux) : nullptr;
        a.idx = indices ? reinterpret_cast<const int64_t *>(aux) : nullptr;
    } else {
        a.chunk = chunk;
        a.mask = mask;
        a.idx = indices;
    }

    if (indices) {
        // Dense tiles pay once the list holds about one parameter in 16 of
        // the span it may address: its scattered updates would then touch
        // most cache lines of the sums, weight sums and counts anyway.  They
        // need whole 16-byte quads (N a multiple of 4, aligned arrays).
        const int64_t span = st.N - offset;
        const bool can_tile = st.N % 4 == 0 && aligned16(st.acc) && aligned16(st.wsum) &&
                              (reinterpret_cast<uintptr_t>(st.count) & 3u) == 0;
        const bool tiled = can_tile && (g_index_tiles == 2 ||
                                        (g_index_tiles == 0 && len >= INDEX_TILES_MIN_LEN && len >= span / 16));
        e = fa::launch_stream_accumulate_indices(a, dtype, tiled, st.list_gate(), st.compute);
    } else {
        const int part = !st.partial ? fa::PART_DENSE : (mask ? fa::PART_MASK : fa::PART_RANGE);
        const bool aligned = (offset % fa::VEC) == 0 && aligned16(a.chunk) &&
                             (!a.mask || (reinterpret_cast<uintptr_t>(a.mask) & 7u) == 0);
        e = fa::launch_stream_accumulate(a, dtype, part, aligned, grid_cap(), STREAM_ACC_RESIDENT, st.compute);
    }
    if (e != hipSuccess)
        return hip_fail(e, "accumulate launch");
    if (slot >= 0) {
        const int rc = st.release(slot);
        if (rc != FA_OK)
            return rc;
    }
    st.clients[client_id] = cl;
    return ok();
}

int fedavg_accumulate_partial(fa_handle h, int client_id, int64_t W, int n_clients,
                              const float *acc_src, const uint32_t *wsum_src,
                              const uint8_t *count_src, int64_t offset, int64_t len)
{
    if (!h)
        return fail(FA_ERR_ARG, "NULL handle");
    fa_stream_state &st = *h;
    {
        const int rc = st.open_call();
        if (rc != FA_OK)
            return rc;
    }
    if (st.finalized)
        return fail(FA_ERR_STATE, "accumulate after finalize");
    if (client_id < 0)
        return fail(FA_ERR_ARG, "client_id must be >= 0");
    if (W < 0 || W >= (1ll << 32))
        return fail(FA_ERR_RANGE, "W=%lld outside [0, 2^32)", (long long)W);
    if (n_clients < 1 || n_clients > FA_MAX_STREAM_CLIENTS)
        return fail(FA_ERR_RANGE, "n_clients=%d outside [1, %d]", n_clients, FA_MAX_STREAM_CLIENTS);
    if (len < 0 || offset < 0 || offset > st.N || len > st.N - offset)
        return fail(FA_ERR_RANGE, "range at %lld of %lld elements outside [0, N=%lld)",
                    (long long)offset, (long long)len, (long long)st.N);
    if (len > 0 && !acc_src)
        return fail(FA_ERR_ARG, "acc_src is NULL");
    if (st.partial && len > 0 && !wsum_src)
        return fail(FA_ERR_ARG, "a partial-mode handle needs wsum_src");
    if (st.partial && st.count && len > 0 && !count_src)
        return fail(FA_ERR_ARG, "a handle with client counts needs count_src");

    auto it = st.clients.find(client_id);
    if (it != st.clients.end() && (it->second.n != W || it->second.members != n_clients))
        return fail(FA_ERR_ARG, "client %d changed its weight or client count", client_id);
    if (W == 0)
        return ok();
    if (it == st.clients.end()) {
        const int rc = st.admit(W, n_clients);
        if (rc != FA_OK)
            return rc;
    }
    fa_stream_state::Client cl =
        it != st.clients.end() ? it->second : fa_stream_state::Client{W, 0, n_clients};
    if (len == 0) {
        st.clients[client_id] = cl;
        return ok();
    }
    {
        const int rc = st.cover(client_id, cl, offset, len);
        if (rc != FA_OK)
            return rc;
    }

    const bool use_wsum = st.partial;
    const bool use_count = st.partial && st.count;
    const Residence res = residence_of(acc_src);
    if (res == Residence::Pageable)
        return fail(FA_ERR_ARG, "acc_src must be pinned host memory or device memory");
    if ((use_wsum && residence_of(wsum_src) != res) || (use_count && residence_of(count_src) != res))
        return fail(FA_ERR_ARG, "wsum_src and count_src must live where acc_src lives");

    fa::StreamArgs a;
    std::memset(&a, 0, sizeof a);
    a.acc = st.acc;
    a.wsum = st.wsum;
    a.count = st.count;
    a.offset = offset;
    a.len = len;
    a.N = st.N;
    a.err = st.err_flag();
    int slot = -1;
    if (res == Residence::PinnedHost) {
        // sums in the slot's value area, weight sums and counts in its aux area
        const size_t vbytes = (size_t)len * 4;
        if (vbytes > (size_t)st.chunk_bytes)
            return fail(FA_ERR_RANGE, "%zu bytes of partial sums exceed chunk_bytes=%lld", vbytes,
                        (long long)st.chunk_bytes);
        const size_t aux_at = round_up((size_t)st.chunk_bytes, 256);
        const size_t cnt_at = aux_at + round_up(vbytes, 256);
        const size_t end = use_count ? cnt_at + (size_t)len : (use_wsum ? aux_at + vbytes : vbytes);
        if (end > st.slot_size)
            return fail(FA_ERR_RANGE, "a partial of %lld parameters does not fit a staging slot of "
                        "%zu bytes", (long long)len, st.slot_size);
        const void *src[3] = {acc_src, use_wsum ? wsum_src : nullptr, use_count ? count_src : nullptr};
        const size_t bytes[3] = {vbytes, use_wsum ? vbytes : 0, use_count ? (size_t)len : 0};
        const size_t at[3] = {0, aux_at, cnt_at};
        slot = st.stage(src, bytes, at, 3);
        if (slot < 0)
            return FA_ERR_HIP; // message recorded by stage()
        a.chunk = st.slot(slot);
        a.src_wsum = reinterpret_cast<const uint32_t *>(st.slot(slot) + aux_at);
        a.src_count = reinterpret_cast<const uint8_t *>(st.slot(slot) + cnt_at);
    } else {
        a.chunk = acc_src;
        a.src_wsum = wsum_src;
        a.src_count = count_src;
    }
    const bool aligned = (offset % fa::VEC) == 0 && aligned16(a.chunk) &&
                         (!use_wsum || aligned16(a.src_wsum)) &&
                         (!use_count || (reinterpret_cast<uintptr_t>(a.src_count) & 7u) == 0);
    hipError_t e =
        fa::launch_stream_merge(a, use_wsum, aligned, grid_cap(), STREAM_MERGE_RESIDENT, st.compute);
    if (e != hipSuccess)
        return hip_fail(e, "merge launch");
    if (slot >= 0) {
        const int rc = st.release(slot);
        if (rc != FA_OK)
            return rc;
    }
    st.clients[client_id] = cl;
    return ok();
}

int fedavg_partial_info(fa_handle h, int64_t *W, int *n_clients)
{
    if (!h)
        return fail(FA_ERR_ARG, "NULL handle");
    if (W)
        *W = (int64_t)h->total_weight();
    if (n_clients)
        *n_clients = (int)h->total_members();
    return ok();
}

int fedavg_finalize(fa_handle h, const void *base, fa_dtype base_dtype, void *out,
                    fa_dtype out_dtype)
{
    if (!h)
        return fail(FA_ERR_ARG, "NULL handle");
    fa_stream_state &st = *h;
    if (!dtype_ok(base_dtype) || !dtype_ok(out_dtype))
        return fail(FA_ERR_DTYPE, "dtypes must be FA_F32 or FA_BF16");
    if (st.N > 0 && !out)
        return fail(FA_ERR_ARG, "out must not be NULL");
    if (st.N > 0 && (st.mode != FA_WEIGHTS || st.partial) && !base)
        return fail(FA_ERR_ARG, "base is required in delta and partial modes");
    if (base && !overlap_ok(out, (size_t)st.N * dsize(out_dtype), base,
                            (size_t)st.N * dsize(base_dtype)))
        return fail(FA_ERR_ARG, "out partially overlaps base");
    for (auto &c : st.clients) {
        if (!st.partial && c.second.covered != st.N)
            return fail(FA_ERR_INCOMPLETE, "client %d covered [0, %lld) of [0, %lld)", c.first,
                        (long long)c.second.covered, (long long)st.N);
    }
    const uint64_t S = st.total_weight();
    // a rejected finalize leaves the handle open for more clients
    if (st.N > 0 && !st.partial && S == 0 && st.mode == FA_WEIGHTS)
        return fail(FA_ERR_ZERO_WEIGHT, "no client was accumulated in dense weights mode");
    st.finalized = true;
    if (st.N == 0)
        return ok();
    hipError_t e;
    if (!st.partial && S == 0) {
        e = fa::launch_convert(base, base_dtype, out, out_dtype, st.N, st.compute);
        return e == hipSuccess ? ok() : hip_fail(e, "convert launch");
    }
    fa::FinalizeArgs a;
    a.acc = st.acc;
    a.wsum = st.wsum;
    a.base = base;
    a.out = out;
    a.N = st.N;
    a.S = (float)S;
    a.zero_fill = st.mode == FA_DELTAS_ZERO_FILL;
    const bool aligned = aligned16(out) && (!base || aligned16(base));
    e = fa::launch_stream_finalize(a, base_dtype, out_dtype,
                                   st.mode == FA_WEIGHTS ? FA_WEIGHTS : FA_DELTAS, st.partial,
                                   aligned, grid_cap(), STREAM_FIN_RESIDENT, st.compute);
    return e == hipSuccess ? ok() : hip_fail(e, "finalize launch");
}

int fedavg_sync(fa_handle h)
{
    if (!h)
        return fail(FA_ERR_ARG, "NULL handle");
    fa_stream_state &st = *h;
    hipError_t e = hipStreamSynchronize(st.copy);
    if (e == hipSuccess)
        e = hipStreamSynchronize(st.compute);
    int flag = 0;
    if (e == hipSuccess)
        e = hipMemcpy(&flag, st.err_flag(), sizeof flag, hipMemcpyDeviceToHost);
    if (e != hipSuccess)
        return hip_fail(e, "sync");
    if (flag != 0)
        return fail(FA_ERR_INDEX, "a chunk held unsorted, duplicate or out-of-range indices");
    return ok();
}

int fedavg_destroy(fa_handle h)
{
    if (!h)
        return ok();
    fa_stream_state *st = h;
    hipError_t e = hipStreamSynchronize(st->copy);
    hipError_t e2 = hipStreamSynchronize(st->compute);
    for (auto ev : st->copy_done)
        if (ev)
            (void)hipEventDestroy(ev);
    for (auto ev : st->slot_free)
        if (ev)
            (void)hipEventDestroy(ev);
    if (st->own_copy && st->copy)
        (void)hipStreamDestroy(st->copy);
    delete st;
    if (e != hipSuccess)
        return hip_fail(e, "destroy");
    if (e2 != hipSuccess)
        return hip_fail(e2, "destroy");
    return ok();
}

// ============================================================ sparse

static int64_t sparse_blocks_for(int64_t N, int64_t tile)
{
    const int64_t tiles = (N + tile - 1) / tile;
    // Many short ranges rather than one per resident slot: workgroups start
    // in range order, so the ones running at any moment read neighbouring
    // stretches of every client's list (measured faster on MI355X than
    // persistent workgroups spread over the whole index space).  Shorter
    // ranges speed the merge up further but cost a boundary search per
    // client and range: at 10^9 parameters and K = 20 (2048-parameter tiles)
    // ranges of 8, 4 and 2 tiles gave 6.87, 6.73 and 6.69-6.76 ms per call
    // (merge 6.76, 6.55, 6.36 ms; searches 0.11, 0.18, 0.33 ms).  Below
    // SPARSE_MIN_RANGES ranges shorter ones keep the GPU filled.
    int64_t want = g_sparse_blocks;
    if (want <= 0)
        want = std::max<int64_t>((tiles + SPARSE_RANGE_TILES - 1) / SPARSE_RANGE_TILES,
                                 std::min<int64_t>(tiles, SPARSE_MIN_RANGES));
    want = std::min<int64_t>(want, SPARSE_MAX_BLOCKS);
    int64_t nb = std::min<int64_t>(tiles, want);
    if (nb < 1)
        nb = 1;
    const int64_t tiles_per_block = (tiles + nb - 1) / nb;
    const int64_t R = tiles_per_block * tile;
    return (N + R - 1) / R;
}

int sparse_workspace_size(int K, int64_t N, size_t *bytes)
{
    if (K < 1 || K > FA_MAX_CLIENTS)
        return fail(FA_ERR_RANGE, "K=%d outside [1, %d]", K, FA_MAX_CLIENTS);
    if (N < 0 || !bytes)
        return fail(FA_ERR_ARG, "need N >= 0 and a result pointer");
    if (N > FA_MAX_N)
        return fail(FA_ERR_RANGE, "N=%lld exceeds 2^40", (long long)N);
    // one list offset per client and range boundary; there are never more
    // ranges than tiles of the smallest tile size
    const int64_t max_ranges =
        std::min<int64_t>(SPARSE_MAX_BLOCKS, std::max<int64_t>(1, (N + SPARSE_MIN_TILE - 1) / SPARSE_MIN_TILE));
    *bytes = HEADER_BYTES + (size_t)K * (size_t)(max_ranges + 1) * sizeof(int64_t);
    return ok();
}

} // extern "C"

// Scratch of the allocation-free sparse merge: the range offsets (and the
// error flag when the caller passes none).  One copy per GPU, held until the
// process ends.  In host code `scratch` names a host-side stand-in, never
// passed to a kernel: the device address comes from hipGetSymbolAddress,
// looked up per device.
constexpr size_t SPARSE_SCRATCH_BYTES = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[SPARSE_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the current device, looked up on the first
// call there; threads that race store the same address.  NULL after a failed
// lookup (recorded as FA_ERR_HIP in *rc).
void *scratch_address(int *rc)
{
    static std::atomic<void *> cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *rc = hip_fail(e, "current device");
        return nullptr;
    }
    if (dev < 0 || dev >= 64) {
        *rc = fail(FA_ERR_RANGE, "device %d: at most 64 devices", dev);
        return nullptr;
    }
    void *p = cache[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            *rc = hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "scratch address");
            return nullptr;
        }
        cache[dev].store(p, std::memory_order_release);
    }
    return p;
}

// Shared body of the sparse merge entry points.  workspace == nullptr with
// use_scratch: the workspace is this device's `scratch`.
int sparse_run(int K, const int64_t *const *idx, const float *const *val, const int64_t *nnz,
               const int64_t *n, int64_t N, fa_mode mode, const float *base, float *out,
               void *counts, fa_count_dtype counts_dtype, uint32_t *wsum, void *workspace,
               size_t workspace_bytes, bool use_scratch, int *err_flag, void *stream)
{
    if (K < 1 || K > FA_MAX_CLIENTS)
        return fail(FA_ERR_RANGE, "K=%d outside [1, %d]", K, FA_MAX_CLIENTS);
    if (!idx || !val || !nnz || !n)
        return fail(FA_ERR_ARG, "idx, val, nnz and n must not be NULL");
    if (N < 0)
        return fail(FA_ERR_ARG, "N is negative");
    if (N > FA_MAX_N)
        return fail(FA_ERR_RANGE, "N=%lld exceeds 2^40", (long long)N);
    if (mode != FA_WEIGHTS && mode != FA_DELTAS && mode != FA_DELTAS_ZERO_FILL)
        return fail(FA_ERR_ARG, "unknown mode %d", (int)mode);
    if (counts_dtype != FA_COUNT_U8 && counts_dtype != FA_COUNT_U32)
        return fail(FA_ERR_DTYPE, "counts dtype must be FA_COUNT_U8 or FA_COUNT_U32");
    if (N > 0 && (!base || !out))
        return fail(FA_ERR_ARG, "base and out are required");
    if (!overlap_ok(out, (size_t)N * 4, base, (size_t)N * 4))
        return fail(FA_ERR_ARG, "out partially overlaps base");

    fa::SparseArgs a;
    std::memset(&a, 0, sizeof a);
    uint64_t S_all = 0; // every client with n_k > 0, also one whose list is empty
    int Kc = 0;
    for (int k = 0; k < K; ++k) {
        if (n[k] < 0 || n[k] > FA_MAX_WEIGHT)
            return fail(FA_ERR_RANGE, "n[%d]=%lld outside [0, 2^24]", k, (long long)n[k]);
        if (nnz[k] < 0)
            return fail(FA_ERR_ARG, "nnz[%d] is negative", k);
        S_all += (uint64_t)n[k];
        if (n[k] == 0 || nnz[k] == 0)
            continue;
        if (!idx[k] || !val[k])
            return fail(FA_ERR_ARG, "idx[%d] or val[%d] is NULL", k, k);
        a.idx[Kc] = idx[k];
        a.val[Kc] = val[k];
        a.nnz[Kc] = nnz[k];
        a.w[Kc] = (float)n[k];
        a.wi[Kc] = (uint32_t)n[k];
        ++Kc;
    }
    if (S_all >= (1ull << 32))
        return fail(FA_ERR_RANGE, "sum of n_k must be below 2^32");
    hipStream_t s = static_cast<hipStream_t>(stream);
    // an empty model has nothing to merge: only the caller's flag is reset,
    // and no workspace is needed
    if (N == 0) {
        if (err_flag) {
            const hipError_t e = fa::launch_fill_u32(err_flag, 1, 0u, s);
            if (e != hipSuccess)
                return hip_fail(e, "flag reset");
        }
        return ok();
    }
    // plan the ranges and check the workspace before anything is enqueued:
    // the offsets kernel writes Kc * (NB + 1) list positions
    const int64_t tile = g_sparse_tile;
    const int64_t NB = sparse_blocks_for(N, tile);
    const int64_t tiles = (N + tile - 1) / tile;
    const int64_t R = ((tiles + NB - 1) / NB) * tile;
    const size_t used = HEADER_BYTES + (size_t)Kc * (size_t)(NB + 1) * sizeof(int64_t);
    if (use_scratch) {
        if (used > SPARSE_SCRATCH_BYTES)
            return fail(FA_ERR_RANGE,
                        "%d contributing clients over %lld ranges need %zu bytes of offsets; the "
                        "allocation-free call holds %zu", Kc, (long long)NB, used,
                        SPARSE_SCRATCH_BYTES);
        int rc = FA_OK;
        workspace = scratch_address(&rc);
        if (!workspace)
            return rc;
        workspace_bytes = SPARSE_SCRATCH_BYTES;
    } else {
        size_t need = 0;
        sparse_workspace_size(K, N, &need);
        if (!workspace || workspace_bytes < need)
            return fail(FA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                        need);
        if (used > workspace_bytes)
            return fail(FA_ERR_WORKSPACE, "workspace has %zu bytes, %lld ranges need %zu",
                        workspace_bytes, (long long)NB, used);
    }
    int *flag = err_flag ? err_flag : static_cast<int *>(workspace);
    hipError_t e = fa::launch_fill_u32(flag, 1, 0u, s);
    if (e != hipSuccess)
        return hip_fail(e, "flag reset");
    a.K = Kc;
    a.NB = (int)NB;
    a.N = N;
    a.R = R;
    a.tile = (int)tile;
    a.offs = reinterpret_cast<int64_t *>(static_cast<char *>(workspace) + HEADER_BYTES);
    a.base = base;
    a.out = out;
    a.counts = counts;
    a.counts_u32 = counts_dtype == FA_COUNT_U32;
    a.wsum = wsum;
    a.mode = mode == FA_WEIGHTS ? FA_WEIGHTS : FA_DELTAS;
    a.zero_fill = mode == FA_DELTAS_ZERO_FILL;
    a.S_all = (float)S_all;
    a.aligned = aligned16(base) && aligned16(out) && (!wsum || aligned16(wsum)) &&
                (!counts || aligned16(counts));
    a.err = flag;
    e = fa::launch_sparse(a, s);
    return e == hipSuccess ? ok() : hip_fail(e, "sparse launch");
}

} // namespace

extern "C" {

int sparse_masked_accumulate(int K, const int64_t *const *idx, const float *const *val,
                             const int64_t *nnz, const int64_t *n, int64_t N, fa_mode mode,
                             const float *base, float *out, void *counts,
                             fa_count_dtype counts_dtype, uint32_t *wsum, void *workspace,
                             size_t workspace_bytes, int *err_flag, void *stream)
{
    return sparse_run(K, idx, val, nnz, n, N, mode, base, out, counts, counts_dtype, wsum, workspace,
                      workspace_bytes, false, err_flag, stream);
}

int sparse_masked_accumulate_noalloc(int K, const int64_t *const *idx, const float *const *val,
                                     const int64_t *nnz, const int64_t *n, int64_t N, fa_mode mode,
                                     const float *base, float *out, void *counts,
                                     fa_count_dtype counts_dtype, uint32_t *wsum, int *err_flag,
                                     void *stream)
{
    return sparse_run(K, idx, val, nnz, n, N, mode, base, out, counts, counts_dtype, wsum, nullptr,
                      0, true, err_flag, stream);
}

// ============================================================ sample allocation

namespace {

double median_of(std::vector<double> v)
{
    std::sort(v.begin(), v.end());
    const size_t m = v.size();
    return m % 2 ? v[m / 2] : (v[m / 2 - 1] + v[m / 2]) / 2.0;
}

} // namespace

int fedavg_controller_step(int P, const double *t, const double *e, const int64_t *n,
                           int64_t total, const fa_controller *c, double *tau_state,
                           double *eps_state, int first_round, int64_t *n_next)
{
    if (P < 1 || !t || !e || !n || !c || !tau_state || !eps_state || !n_next)
        return fail(FA_ERR_ARG, "need P >= 1 and every array");
    if (total < P)
        return fail(FA_ERR_RANGE, "total=%lld is below the %d participants", (long long)total, P);
    if (!(c->ema > 0.0 && c->ema <= 1.0) || !(c->deadband >= 0.0) || !(c->w_time >= 0.0) ||
        !(c->w_energy >= 0.0) || (c->w_time == 0.0 && c->w_energy == 0.0))
        return fail(FA_ERR_ARG, "need 0 < ema <= 1, deadband >= 0, weights >= 0 and not both 0");
    int64_t nsum = 0;
    for (int i = 0; i < P; ++i) {
        if (n[i] <= 0 || !(t[i] >= 0.0) || !(e[i] >= 0.0))
            return fail(FA_ERR_ARG, "participant %d: need n > 0, time and energy >= 0", i);
        nsum += n[i];
    }
    // per-sample costs, smoothed
    std::vector<double> tau(P), eps(P);
    for (int i = 0; i < P; ++i) {
        tau[i] = t[i] / (double)n[i];
        eps[i] = e[i] / (double)n[i];
        if (!first_round) {
            tau[i] = c->ema * tau[i] + (1.0 - c->ema) * tau_state[i];
            eps[i] = c->ema * eps[i] + (1.0 - c->ema) * eps_state[i];
        }
    }
    // combined cost, each term normalised by its median
    std::vector<double> cost(P, 0.0);
    if (c->w_time != 0.0) {
        const double mt = median_of(tau);
        if (!(mt > 0.0))
            return fail(FA_ERR_ARG, "the median time cost is zero");
        for (int i = 0; i < P; ++i)
            cost[i] += c->w_time * tau[i] / mt;
    }
    if (c->w_energy != 0.0) {
        const double me = median_of(eps);
        if (!(me > 0.0))
            return fail(FA_ERR_ARG, "the median energy cost is zero");
        for (int i = 0; i < P; ++i)
            cost[i] += c->w_energy * eps[i] / me;
    }
    std::vector<double> inv(P);
    double z = 0.0;
    for (int i = 0; i < P; ++i) {
        if (!(cost[i] > 0.0))
            return fail(FA_ERR_ARG, "participant %d has a cost that is not positive", i);
        inv[i] = 1.0 / cost[i];
    }
    for (int i = 0; i < P; ++i)
        z += inv[i];
    // samples in inverse proportion to the cost: largest remainder
    std::vector<double> target(P);
    std::vector<int64_t> cnt(P);
    int64_t given = 0;
    for (int i = 0; i < P; ++i) {
        target[i] = (double)total * (inv[i] / z);
        cnt[i] = (int64_t)std::floor(target[i]);
        given += cnt[i];
    }
    std::vector<int> order(P);
    for (int i = 0; i < P; ++i)
        order[i] = i;
    std::sort(order.begin(), order.end(), [&](int a, int b) {
        const double fa_ = target[a] - (double)cnt[a], fb_ = target[b] - (double)cnt[b];
        return fa_ != fb_ ? fa_ > fb_ : a < b;
    });
    for (int64_t j = 0; j < total - given && j < P; ++j)
        cnt[order[j]] += 1;
    // everyone keeps a sample, taken from the largest count (lowest index)
    for (int i = 0; i < P; ++i) {
        while (cnt[i] < 1) {
            int big = 0;
            for (int q = 1; q < P; ++q)
                if (cnt[q] > cnt[big])
                    big = q;
            cnt[big] -= 1;
            cnt[i] += 1;
        }
    }
    // deadband: keep the current counts when every change is within it
    bool keep = nsum == total;
    for (int i = 0; i < P && keep; ++i)
        keep = std::fabs((double)(cnt[i] - n[i])) <= c->deadband * (double)n[i];
    for (int i = 0; i < P; ++i) {
        n_next[i] = keep ? n[i] : cnt[i];
        tau_state[i] = tau[i];
        eps_state[i] = eps[i];
    }
    return ok();
}

// ============================================================ top-k selection

// One workgroup per 8192-element tile, and a launch holds at most 2^32 - 1
// work-items: 2^36 elements (256 GB of fp32) is the most top-k takes.
constexpr int64_t TOPK_MAX_N = 1ll << 36;

int topk_workspace_size(fa_dtype dtype, int64_t N, int64_t k, size_t *bytes)
{
    if (!bytes)
        return fail(FA_ERR_ARG, "need a result pointer");
    if (!dtype_ok(dtype))
        return fail(FA_ERR_DTYPE, "dtype must be FA_F32 or FA_BF16");
    if (N < 0 || k < 0 || k > N)
        return fail(FA_ERR_RANGE, "need 0 <= k <= N (k=%lld, N=%lld)", (long long)k, (long long)N);
    if (N > TOPK_MAX_N)
        return fail(FA_ERR_RANGE, "N=%lld is too large (at most 2^36)", (long long)N);
    *bytes = fa::topk_workspace_bytes(dtype, N, k);
    return ok();
}

int topk_select(const void *x, fa_dtype dtype, int64_t N, int64_t k, int64_t *idx_out,
                float *val_out, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!dtype_ok(dtype))
        return fail(FA_ERR_DTYPE, "x must be FA_F32 or FA_BF16");
    if (N < 0 || k < 0 || k > N)
        return fail(FA_ERR_RANGE, "need 0 <= k <= N (k=%lld, N=%lld)", (long long)k, (long long)N);
    if (k == 0)
        return ok();
    if (!x || !idx_out || !val_out || !workspace)
        return fail(FA_ERR_ARG, "x, idx_out, val_out and workspace are required");
    if (N > TOPK_MAX_N)
        return fail(FA_ERR_RANGE, "N=%lld is too large (at most 2^36)", (long long)N);
    const size_t need = fa::topk_workspace_bytes(dtype, N, k);
    if (workspace_bytes < need)
        return fail(FA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    if ((reinterpret_cast<uintptr_t>(workspace) & 15u) != 0 ||
        (reinterpret_cast<uintptr_t>(idx_out) & 7u) != 0 ||
        (reinterpret_cast<uintptr_t>(val_out) & 3u) != 0)
        return fail(FA_ERR_ARG, "workspace must be 16-byte aligned, idx_out 8 and val_out 4");
    const size_t xbytes = (size_t)N * dsize(dtype);
    if (!overlap_ok(idx_out, (size_t)k * 8, x, xbytes) || !overlap_ok(val_out, (size_t)k * 4, x, xbytes) ||
        idx_out == x || val_out == x)
        return fail(FA_ERR_ARG, "outputs must not overlap the input");
    hipError_t e = fa::launch_topk(x, dtype, N, k, idx_out, val_out, workspace, cu_count(),
                                   static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "top-k launch");
}

// ============================================================ checksum

int fedavg_checksum(const void *buf, int64_t count, fa_dtype dtype, uint64_t *hash_dev, void *stream)
{
    if (!hash_dev || (count > 0 && !buf) || count < 0)
        return fail(FA_ERR_ARG, "need a hash pointer, a buffer and count >= 0");
    if (count > FA_MAX_N)
        return fail(FA_ERR_RANGE, "count=%lld exceeds 2^40", (long long)count);
    if (!dtype_ok(dtype))
        return fail(FA_ERR_DTYPE, "dtype must be FA_F32 or FA_BF16");
    hipError_t e = fa::launch_checksum(buf, count, dtype, hash_dev, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "checksum launch");
}

int fedavg_sum_workspace_size(int64_t count, size_t *bytes)
{
    if (!bytes || count < 0)
        return fail(FA_ERR_ARG, "need count >= 0 and a result pointer");
    if (count > FA_MAX_N)
        return fail(FA_ERR_RANGE, "count=%lld exceeds 2^40", (long long)count);
    *bytes = (size_t)((count + fa::SUM_TILE - 1) / fa::SUM_TILE) * sizeof(double);
    return ok();
}

int fedavg_checksum_sum(const void *buf, int64_t count, fa_dtype dtype, uint64_t *hash_dev,
                        double *sum_dev, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!sum_dev || (count > 0 && !buf) || count < 0)
        return fail(FA_ERR_ARG, "need a sum pointer, a buffer and count >= 0");
    if (count > FA_MAX_N)
        return fail(FA_ERR_RANGE, "count=%lld exceeds 2^40", (long long)count);
    if (!dtype_ok(dtype))
        return fail(FA_ERR_DTYPE, "dtype must be FA_F32 or FA_BF16");
    size_t need = 0;
    fedavg_sum_workspace_size(count, &need);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(FA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 7u) != 0)
        return fail(FA_ERR_ARG, "workspace must be 8-byte aligned");
    if ((reinterpret_cast<uintptr_t>(sum_dev) & 7u) != 0 ||
        (hash_dev && (reinterpret_cast<uintptr_t>(hash_dev) & 7u) != 0))
        return fail(FA_ERR_ARG, "sum_dev and hash_dev must be 8-byte aligned");
    // the tile sums are written while the buffer is read, and the results
    // after: none of them may share bytes with the buffer or the tile sums
    auto apart = [](const void *a, size_t an, const void *b, size_t bn) {
        const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
        return !a || !b || an == 0 || bn == 0 || a0 + an <= b0 || b0 + bn <= a0;
    };
    const size_t bbytes = (size_t)count * dsize(dtype);
    if (!apart(workspace, need, buf, bbytes) || !apart(sum_dev, 8, buf, bbytes) ||
        !apart(hash_dev, 8, buf, bbytes) || !apart(sum_dev, 8, workspace, need) ||
        !apart(hash_dev, 8, workspace, need) || !apart(hash_dev, 8, sum_dev, 8))
        return fail(FA_ERR_ARG, "the buffer, the workspace and the results must not overlap");
    // workgroups walk the tiles: a few per CU by default
    const int64_t cap = grid_cap() > 0 ? grid_cap() : (int64_t)cu_count() * 32;
    hipError_t e = fa::launch_checksum_sum(buf, count, dtype, hash_dev, sum_dev,
                                           static_cast<double *>(workspace), cap,
                                           static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "checksum and sum launch");
}

} // extern "C"
