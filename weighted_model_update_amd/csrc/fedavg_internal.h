// Internal interface between the host library (fedavg_api.hip) and the
// gfx950 kernels (fedavg_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fedavg.h"

namespace fa {

enum { DT_F32 = FA_F32, DT_BF16 = FA_BF16 };
enum { MODE_WEIGHTS = FA_WEIGHTS, MODE_DELTAS = FA_DELTAS };

// Elements handled per thread per step on the vector paths: 8 bf16 are one
// 16-byte load, 8 fp32 are two.
constexpr int VEC = 8;
constexpr int TAB_SEGS = 512; // segment tables up to this size are staged whole in LDS

// ---------------------------------------------------------------- resident
struct DenseArgs {
    const void *x[FA_MAX_CLIENTS]; // contributing clients only (n_k > 0)
    float w[FA_MAX_CLIENTS];       // fp32(n_k), exact; -0 past K
    int K;                         // number of contributing clients
    int64_t N;
    const void *base;
    void *out;
    float S; // fp32(sum n_k)
};

struct MaskedArgs {
    const void *x[FA_MAX_CLIENTS];
    float w[FA_MAX_CLIENTS];
    uint32_t wi[FA_MAX_CLIENTS];
    int row[FA_MAX_CLIENTS]; // row of each contributing client in `present`
    int K;
    int T;
    int64_t N;
    int64_t vpb; // vectors per block
    const int64_t *bounds;
    const uint8_t *present;
    const void *base;
    void *out;
    int zero_fill; // divide by S_all (all clients' weight) instead of W_i
    float S_all;
};

// ---------------------------------------------------------------- streaming
enum { PART_DENSE = 0, PART_RANGE = 1, PART_MASK = 2 };

struct StreamArgs {
    const void *chunk;
    const uint8_t *mask;
    const int64_t *idx;
    float *acc;
    uint32_t *wsum;
    uint8_t *count;
    int64_t offset;
    int64_t len;
    int64_t N;
    float w;
    uint32_t wi;
    int *err;
    // merging another accumulator's partial sums: its per-parameter weight
    // sums and client counts (chunk then holds its fp32 sums)
    const uint32_t *src_wsum;
    const uint8_t *src_count;
    // client-at-a-time sparse accumulate: when set, the scatter kernel runs
    // only if *gate is nonzero (the list failed the tiled path's check)
    const int *gate;
};

struct FinalizeArgs {
    const float *acc;
    const uint32_t *wsum;
    const void *base;
    void *out;
    int64_t N;
    float S;
    int zero_fill; // partial mode: divide by S instead of the weight sums
};

// ---------------------------------------------------------------- sparse
constexpr int SP_GROUP = 8;     // clients whose batches are loaded together
constexpr int SP_DEFAULT_TILE = 2048; // parameters per LDS tile (512 ... 8192, powers of 2)

struct SparseArgs {
    const int64_t *idx[FA_MAX_CLIENTS];
    const float *val[FA_MAX_CLIENTS];
    int64_t nnz[FA_MAX_CLIENTS];
    float w[FA_MAX_CLIENTS];
    uint32_t wi[FA_MAX_CLIENTS];
    int K;
    int NB;    // blocks (parameter ranges)
    int64_t N;
    int64_t R; // parameters per block range, a multiple of the tile
    int tile;  // parameters per LDS tile: 512, 1024, 2048, 4096 or 8192
    int64_t *offs; // [K][NB+1] first list position at or after each range start
    const float *base;
    float *out;
    void *counts;
    int counts_u32;
    uint32_t *wsum;
    int mode;
    int aligned; // base/out/counts/wsum allow the 8-wide finalize
    int *err;
    int zero_fill; // divide by S_all (all clients' weight) instead of W_i
    float S_all;
};

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.  `grid_cap` bounds the number
// of workgroups of grid-stride kernels (0: one 8-element group per thread);
// `resident` caps the workgroups resident per CU (0: hardware limit).
hipError_t launch_dense(const DenseArgs &a, int xdt, int odt, int bdt, int mode, bool aligned,
                        int64_t grid_cap, int resident, hipStream_t s);
hipError_t launch_masked(const MaskedArgs &a, int xdt, int odt, int bdt, int mode, bool aligned,
                         hipStream_t s);
hipError_t launch_stream_accumulate(const StreamArgs &a, int dt, int part, bool aligned,
                                    int64_t grid_cap, int resident, hipStream_t s);
// Client-at-a-time sparse accumulate.  tiled: check the list, and if it is
// sorted and inside the accumulator apply it over dense tiles, else scatter
// it; gate is a device word of scratch the tiled path needs.
hipError_t launch_stream_accumulate_indices(const StreamArgs &a, int dt, bool tiled, int *gate, hipStream_t s);
// Parameters per tile of the tiled index accumulate (fp32 sums, weight sums
// and counts of one tile are read and written whole).
constexpr int IT_TILE = 2048;
hipError_t launch_stream_merge(const StreamArgs &a, bool partial, bool aligned, int64_t cap,
                               int resident, hipStream_t s);
hipError_t launch_stream_finalize(const FinalizeArgs &a, int bdt, int odt, int mode, int partial,
                                  bool aligned, int64_t grid_cap, int resident, hipStream_t s);
int sparse_resident_blocks_per_cu(int tile);
hipError_t launch_sparse(const SparseArgs &a, hipStream_t s);
// client-side top-k selection (topk.hip)
constexpr int TK_TILE = 8192; // elements per tile of the count and write passes
size_t topk_workspace_bytes(int dt, int64_t N, int64_t k);
void topk_set_sampled(int on); // 0: always the full three-pass path
hipError_t launch_topk(const void *x, int dt, int64_t N, int64_t k, int64_t *idx_out,
                       float *val_out, void *ws, int cus, hipStream_t s);
hipError_t launch_checksum(const void *buf, int64_t count, int dt, uint64_t *hash,
                           hipStream_t s);
// Elements per tile sum, and the threads that add the tile sums.
constexpr int SUM_TILE = 8192;
constexpr int SUM_FINISH_THREADS = 1024;
hipError_t launch_checksum_sum(const void *buf, int64_t count, int dt, uint64_t *hash, double *sum,
                               double *part, int64_t cap, hipStream_t s);
hipError_t launch_fill_u32(void *p, int64_t words, uint32_t value, hipStream_t s);
// p must be 4-byte aligned; writes exactly `bytes` bytes.
hipError_t launch_fill_bytes(void *p, int64_t bytes, uint8_t value, hipStream_t s);
hipError_t launch_convert(const void *src, int sdt, void *dst, int ddt, int64_t N, hipStream_t s);

} // namespace fa
