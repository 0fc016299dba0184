/*
 * FedAvg aggregation oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow CPU statement of what server-side federated averaging
 * computes.  Only the test suite, the smoke check and the bench's CPU-baseline
 * leg may load this library; the product path never does.  It shares no code
 * with the HIP library.
 *
 * What is computed, and where it comes from:
 *
 *  - The server combines the clients' models either as a plain average or
 *    weighted by what each client contributed ("NVIDIA Clara implements
 *    federated learning", epnc.co.kr, introduction and the server-side
 *    workflow section, which names a weighted aggregation algorithm).  The
 *    weight of client k is its sample count n_k, which each participant
 *    reports per round (gist.science summary of the measurement-based adaptive
 *    data partitioning paper, section "The adaptive controller",
 *    "Measurement").  So for every parameter i
 *
 *        out_i = sum_{k in C_i} n_k * x_{k,i} / W_i,   W_i = sum_{k in C_i} n_k
 *
 *    with C_i the clients (n_k > 0) that sent parameter i.  In delta mode the
 *    clients send deltas and out_i = base_i + that weighted mean.
 *
 *  - Clients may update only some model components; the update contract says
 *    which, and component updates are averaged over the clients that sent them
 *    ("Building Federated Multimodal AI Workflows with NVIDIA FLARE",
 *    ai-thai.com, sections "Client Update Contract" and the FedUMM
 *    adapter-only example).  Clients may also share only part of their weight
 *    update, each choosing the fraction (Clara page, introduction and
 *    client-side workflow section).  Hence C_i depends on i, and a parameter
 *    no contributing client sent keeps the global value: out_i = base_i.
 *
 *  - A client whose weight is zero contributes nothing (the Ulysses sequence
 *    parallelism page, section "Automatic weighted loss aggregation", makes
 *    the same point for ranks holding only padding).
 *
 *  - Weights are stored in fp32 and rounded to nearest-even, never
 *    stochastically ("NVFP4 training with JAX and MaxText", ai-thai.com,
 *    training-recipe section on stochastic rounding and the data-flow figure
 *    of a linear layer with fp32 master weights).  The oracle therefore returns
 *    ref32_i = round_to_nearest_fp32(exact value); bf16 outputs are compared
 *    against it.
 *
 * Arithmetic: every client value has at most 24 significant bits and every
 * n_k fits in 24 bits, so each product n_k * x_{k,i} is exact in fp64.  The
 * fp64 sum of at most 64 such products is within 64 * 2^-53 * M_i of the
 * exact sum, where M_i = |base_i| + sum n_k |x_{k,i}| / W_i is also returned
 * (the scale of the forward error of any floating-point weighted sum).  The
 * result is rounded once to fp32 (after an fp64 add of the base in delta
 * mode).  The exact-rational brute force in oracle/exact.py pins this.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/*
 * Threads.  The per-parameter loops below run in OpenMP threads, each
 * parameter on one thread with its own arithmetic exactly as written (no
 * parameter's result depends on another's), so the thread count changes the
 * time only.  orc_set_threads(t) sets it (t <= 0 keeps the current one) and
 * returns the count the loops use.
 */
int orc_set_threads(int t)
{
    if (t > 0)
        omp_set_num_threads(t);
    return omp_get_max_threads();
}

enum { ORC_F32 = 0, ORC_BF16 = 1 };
enum { ORC_WEIGHTS = 0, ORC_DELTAS = 1, ORC_DELTAS_ZERO_FILL = 2 };
enum {
    ORC_OK = 0,
    ORC_ERR_ARG = -1,
    ORC_ERR_ZERO_WEIGHT = -4,
    ORC_ERR_INDEX = -7,
    ORC_ERR_NOMEM = -10
};

/* Value of element i of a buffer of the given type, widened exactly. */
static double value_at(const void *buf, int dtype, int64_t i)
{
    if (dtype == ORC_F32)
        return (double)((const float *)buf)[i];
    /* bf16 is the upper half of an IEEE binary32 bit pattern */
    uint32_t bits = ((uint32_t)((const uint16_t *)buf)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static int dtype_ok(int d) { return d == ORC_F32 || d == ORC_BF16; }

/*
 * Resolve one parameter from its per-client sums.
 *   s = sum n_k x_k, m = sum n_k |x_k|, W = sum n_k over the senders,
 *   S = sum n_k over every client with n_k > 0.
 * Zero-fill delta mode reads partial sharing the other way: a client that
 * did not send a parameter counts as having sent a zero delta for it, so the
 * mean is taken over all clients, sum n_k d_k / S (parameters nobody sent
 * still keep base_i exactly).
 */
static int resolve(double s, double m, uint64_t W, uint64_t S, int mode, const void *base,
                   int base_dtype, int64_t i, float *ref32, double *mag)
{
    double b = base ? value_at(base, base_dtype, i) : 0.0;
    if (W == 0) {
        /* nobody sent this parameter: the global value is kept as it is */
        if (!base)
            return ORC_ERR_ZERO_WEIGHT;
        *ref32 = (float)b;
        *mag = fabs(b);
        return ORC_OK;
    }
    const double D = (mode == ORC_DELTAS_ZERO_FILL) ? (double)S : (double)W;
    double mean = s / D;
    double r = (mode == ORC_WEIGHTS) ? mean : b + mean;
    *ref32 = (float)r; /* one rounding to nearest-even */
    *mag = (mode == ORC_WEIGHTS ? 0.0 : fabs(b)) + m / D;
    return ORC_OK;
}

/*
 * Weighted average over an explicit sent relation.
 *   x[k]      client k's N values (type x_dtype)
 *   n[k]      client k's sample count, >= 0
 *   sent      NULL (every client sent every parameter) or K arrays of N bytes
 *   base      N values of type base_dtype, or NULL (only allowed when every
 *             parameter has a sender in weights mode)
 * Outputs (N each): ref32, mag; count and wsum may be NULL.
 */
int orc_weighted_average(int K, const void *const *x, int x_dtype, const int64_t *n,
                         const uint8_t *const *sent, int64_t N, int mode,
                         const void *base, int base_dtype, float *ref32, double *mag,
                         uint32_t *count, uint64_t *wsum)
{
    if (K < 1 || N < 0 || !x || !n || !ref32 || !mag || !dtype_ok(x_dtype))
        return ORC_ERR_ARG;
    if (mode != ORC_WEIGHTS && mode != ORC_DELTAS && mode != ORC_DELTAS_ZERO_FILL)
        return ORC_ERR_ARG;
    if (base && !dtype_ok(base_dtype))
        return ORC_ERR_ARG;
    if (mode != ORC_WEIGHTS && !base)
        return ORC_ERR_ARG;
    uint64_t S = 0;
    for (int k = 0; k < K; ++k) {
        if (n[k] < 0 || (n[k] > 0 && !x[k]))
            return ORC_ERR_ARG;
        S += (uint64_t)n[k];
    }

    int status = ORC_OK;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N; ++i) {
        double s = 0.0, m = 0.0;
        uint64_t W = 0;
        uint32_t c = 0;
        for (int k = 0; k < K; ++k) {
            if (n[k] == 0)
                continue;
            if (sent && !sent[k][i])
                continue;
            double v = value_at(x[k], x_dtype, i);
            s += (double)n[k] * v;
            m += (double)n[k] * fabs(v);
            W += (uint64_t)n[k];
            c += 1;
        }
        int rc = resolve(s, m, W, S, mode, base, base_dtype, i, &ref32[i], &mag[i]);
        if (rc != ORC_OK) {
#pragma omp atomic write
            status = rc;
        }
        if (count)
            count[i] = c;
        if (wsum)
            wsum[i] = W;
    }
    return status;
}

/* First position j of the sorted a[0..len) with a[j] >= v. */
static int64_t lower_bound_i64(const int64_t *a, int64_t len, int64_t v)
{
    int64_t lo = 0, hi = len;
    while (lo < hi) {
        int64_t mid = lo + (hi - lo) / 2;
        if (a[mid] < v)
            lo = mid + 1;
        else
            hi = mid;
    }
    return lo;
}

/*
 * Sparse partial sharing: client k sends nnz[k] (index, value) pairs with
 * strictly increasing indices below N.  Parameters a client did not send are
 * not part of its contribution.  Accumulation runs client by client.
 */
int orc_sparse_average(int K, const int64_t *const *idx, const float *const *val,
                       const int64_t *nnz, const int64_t *n, int64_t N, int mode,
                       const float *base, float *ref32, double *mag, uint32_t *count,
                       uint64_t *wsum)
{
    if (K < 1 || N < 0 || !idx || !val || !nnz || !n || !ref32 || !mag)
        return ORC_ERR_ARG;
    if (mode != ORC_WEIGHTS && mode != ORC_DELTAS && mode != ORC_DELTAS_ZERO_FILL)
        return ORC_ERR_ARG;
    if (mode != ORC_WEIGHTS && !base)
        return ORC_ERR_ARG;
    uint64_t S = 0;
    for (int k = 0; k < K; ++k) {
        if (n[k] < 0 || nnz[k] < 0 || (nnz[k] > 0 && (!idx[k] || !val[k])))
            return ORC_ERR_ARG;
        S += (uint64_t)n[k];
    }

    double *s = calloc((size_t)(N ? N : 1), sizeof(double));
    double *m = calloc((size_t)(N ? N : 1), sizeof(double));
    uint64_t *W = calloc((size_t)(N ? N : 1), sizeof(uint64_t));
    uint32_t *c = calloc((size_t)(N ? N : 1), sizeof(uint32_t));
    int rc = ORC_OK;
    if (!s || !m || !W || !c) {
        rc = ORC_ERR_NOMEM;
        goto done;
    }
    /* every list checked whole, one client per thread */
    int bad = 0;
    const int Kv = rc == ORC_OK ? K : 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int k = 0; k < Kv; ++k) {
        if (n[k] == 0)
            continue;
        for (int64_t j = 0; j < nnz[k]; ++j) {
            int64_t i = idx[k][j];
            if (i < 0 || i >= N || (j > 0 && i <= idx[k][j - 1])) {
                bad = 1;
                break;
            }
        }
    }
    if (bad)
        rc = ORC_ERR_INDEX;
    /* client by client in order for every parameter; the parameters are
       split into blocks, one thread per block, each block visiting every
       client's entries inside it */
    const int64_t B = (int64_t)1 << 16;
    const int64_t nb = rc == ORC_OK ? (N + B - 1) / B : 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < nb; ++b) {
        const int64_t lo = b * B, hi = lo + B < N ? lo + B : N;
        for (int k = 0; k < K; ++k) {
            if (n[k] == 0)
                continue;
            for (int64_t j = lower_bound_i64(idx[k], nnz[k], lo); j < nnz[k] && idx[k][j] < hi; ++j) {
                int64_t i = idx[k][j];
                double v = (double)val[k][j];
                s[i] += (double)n[k] * v;
                m[i] += (double)n[k] * fabs(v);
                W[i] += (uint64_t)n[k];
                c[i] += 1;
            }
        }
    }
    int status = ORC_OK;
    const int64_t nfin = rc == ORC_OK ? N : 0;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nfin; ++i) {
        int r = resolve(s[i], m[i], W[i], S, mode, base, ORC_F32, i, &ref32[i], &mag[i]);
        if (r != ORC_OK) {
#pragma omp atomic write
            status = r;
        }
        if (count)
            count[i] = c[i];
        if (wsum)
            wsum[i] = W[i];
    }
    if (rc == ORC_OK)
        rc = status;
done:
    free(s);
    free(m);
    free(W);
    free(c);
    return rc;
}

/* Position of i in the sorted list a[0..len), or -1 if absent. */
static int64_t find_sorted(const int64_t *a, int64_t len, int64_t i)
{
    int64_t lo = 0, hi = len;
    while (lo < hi) {
        int64_t mid = lo + (hi - lo) / 2;
        if (a[mid] < i)
            lo = mid + 1;
        else
            hi = mid;
    }
    return (lo < len && a[lo] == i) ? lo : -1;
}

/*
 * The same definition evaluated only at the parameters listed in at[0..S):
 * for each one, every client's list is searched for it.  Does not re-check
 * that the lists are sorted (the full version above does).
 */
int orc_sparse_average_at(int K, const int64_t *const *idx, const float *const *val,
                          const int64_t *nnz, const int64_t *n, int64_t N, int mode,
                          const float *base, int64_t S, const int64_t *at, float *ref32,
                          double *mag, uint32_t *count, uint64_t *wsum)
{
    if (K < 1 || N < 0 || S < 0 || !idx || !val || !nnz || !n || !at || !ref32 || !mag)
        return ORC_ERR_ARG;
    if (mode != ORC_WEIGHTS && mode != ORC_DELTAS && mode != ORC_DELTAS_ZERO_FILL)
        return ORC_ERR_ARG;
    if (mode != ORC_WEIGHTS && !base)
        return ORC_ERR_ARG;
    uint64_t Sall = 0; /* total weight of the clients, for zero-fill mode */
    for (int k = 0; k < K; ++k)
        if (n[k] > 0)
            Sall += (uint64_t)n[k];
    for (int64_t q = 0; q < S; ++q)
        if (at[q] < 0 || at[q] >= N)
            return ORC_ERR_ARG;
    int status = ORC_OK;
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < S; ++q) {
        int64_t i = at[q];
        double s = 0.0, m = 0.0;
        uint64_t W = 0;
        uint32_t c = 0;
        for (int k = 0; k < K; ++k) {
            if (n[k] <= 0)
                continue;
            int64_t j = find_sorted(idx[k], nnz[k], i);
            if (j < 0)
                continue;
            double v = (double)val[k][j];
            s += (double)n[k] * v;
            m += (double)n[k] * fabs(v);
            W += (uint64_t)n[k];
            c += 1;
        }
        /* base is indexed by parameter, so resolve against base[i] */
        int rc = resolve(s, m, W, Sall, mode, base, ORC_F32, i, &ref32[q], &mag[q]);
        if (rc != ORC_OK) {
#pragma omp atomic write
            status = rc;
        }
        if (count)
            count[q] = c;
        if (wsum)
            wsum[q] = W;
    }
    return status;
}

/*
 * fp32 -> bf16, round to nearest with ties to even, from the formats'
 * definition: bf16 keeps the sign, the 8 exponent bits and the top 7 fraction
 * bits of binary32.  The 16 dropped bits decide: above half an ulp rounds up,
 * below rounds down, exactly half rounds to the even result.  A carry out of
 * the fraction increments the exponent (the largest finite values round to
 * infinity).  NaN stays NaN (quiet, same sign).
 */
static uint16_t round1_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t exp_bits = (u >> 23) & 0xFFu;
    uint32_t frac = u & 0x7FFFFFu;
    if (exp_bits == 0xFFu && frac != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t hi = u >> 16;
    uint32_t lo = u & 0xFFFFu;
    if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u)))
        hi += 1;
    return (uint16_t)hi;
}

void orc_round_to_bf16(const float *in, uint16_t *out, int64_t count)
{
#pragma omp parallel for schedule(static) if (count > 65536)
    for (int64_t i = 0; i < count; ++i)
        out[i] = round1_bf16(in[i]);
}

/*
 * fp32 mirror of the rounding order the library states for every
 * aggregation path, so that GPU results can be checked bit for bit (the fp64
 * weighted average above is the definition; this is one particular fp32
 * evaluation of it).  For each parameter: acc = +0; for each client in
 * order with n_k > 0 that sent the parameter, acc = fmaf((float)n_k, x,
 * acc), one fused rounding; q = acc / (float)D, an IEEE fp32 division, with
 * D = W (or S, every client with n_k > 0, in zero-fill mode); the delta
 * modes add the base in fp32; the result is rounded to nearest-even into
 * the output type.  A parameter nobody sent takes the base, rounded the
 * same way.  x, base: as for orc_weighted_average; out: N elements of
 * out_dtype (fp32, or bf16 bits).
 */
int orc_mirror_f32(int K, const void *const *x, int x_dtype, const int64_t *n,
                   const uint8_t *const *sent, int64_t N, int mode, const void *base,
                   int base_dtype, int out_dtype, void *out)
{
    if (K < 1 || N < 0 || !x || !n || !out || !dtype_ok(x_dtype) || !dtype_ok(out_dtype))
        return ORC_ERR_ARG;
    if (mode != ORC_WEIGHTS && mode != ORC_DELTAS && mode != ORC_DELTAS_ZERO_FILL)
        return ORC_ERR_ARG;
    if ((mode != ORC_WEIGHTS && !base) || (base && !dtype_ok(base_dtype)))
        return ORC_ERR_ARG;
    uint64_t S = 0;
    for (int k = 0; k < K; ++k) {
        if (n[k] < 0 || (n[k] > 0 && !x[k]))
            return ORC_ERR_ARG;
        S += (uint64_t)n[k];
    }
    int status = ORC_OK;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N; ++i) {
        float acc = 0.0f;
        uint64_t W = 0;
        for (int k = 0; k < K; ++k) {
            if (n[k] == 0 || (sent && !sent[k][i]))
                continue;
            acc = fmaf((float)n[k], (float)value_at(x[k], x_dtype, i), acc);
            W += (uint64_t)n[k];
        }
        float r;
        if (W == 0) {
            if (!base) {
#pragma omp atomic write
                status = ORC_ERR_ZERO_WEIGHT;
                continue;
            }
            r = (float)value_at(base, base_dtype, i);
        } else {
            const float D = (float)(mode == ORC_DELTAS_ZERO_FILL ? S : W);
            const float q = acc / D;
            r = (mode == ORC_WEIGHTS) ? q : (float)value_at(base, base_dtype, i) + q;
        }
        if (out_dtype == ORC_F32)
            ((float *)out)[i] = r;
        else
            ((uint16_t *)out)[i] = round1_bf16(r);
    }
    return status;
}

/*
 * The same fp32 rounding order for sparse (index, value) lists, over the
 * window [first, first + len) of the parameters: client by client in list
 * order, acc_i = fmaf((float)n_k, v, acc_i) from +0 for every entry of the
 * window, W_i += n_k; then each parameter as in orc_mirror_f32 (W_i == 0:
 * base_i; else q = acc_i / (float)D, D = W_i, or S -- every client with
 * n_k > 0 -- in zero-fill mode; weights mode q, delta modes base_i + q in
 * fp32).  idx[k], val[k]: the entries of client k inside the window
 * (nnz[k] of them, strictly increasing global indices), base/out/count/wsum:
 * len elements for the window (base required, as in the library's sparse
 * call; count, wsum nullable).
 */
int orc_sparse_mirror_f32(int K, const int64_t *const *idx, const float *const *val,
                          const int64_t *nnz, const int64_t *n, int64_t first, int64_t len,
                          int mode, const float *base, float *out, uint32_t *count,
                          uint64_t *wsum)
{
    if (K < 1 || first < 0 || len < 0 || !idx || !val || !nnz || !n || !out)
        return ORC_ERR_ARG;
    if (mode != ORC_WEIGHTS && mode != ORC_DELTAS && mode != ORC_DELTAS_ZERO_FILL)
        return ORC_ERR_ARG;
    if (!base)
        return ORC_ERR_ARG;
    uint64_t S = 0;
    for (int k = 0; k < K; ++k) {
        if (n[k] < 0 || nnz[k] < 0 || (nnz[k] > 0 && (!idx[k] || !val[k])))
            return ORC_ERR_ARG;
        S += (uint64_t)n[k];
        for (int64_t j = 0; j < nnz[k]; ++j)
            if (idx[k][j] < first || idx[k][j] >= first + len || (j > 0 && idx[k][j] <= idx[k][j - 1]))
                return ORC_ERR_INDEX;
    }
    float *acc = calloc((size_t)(len ? len : 1), sizeof(float));
    uint64_t *W = calloc((size_t)(len ? len : 1), sizeof(uint64_t));
    uint32_t *c = calloc((size_t)(len ? len : 1), sizeof(uint32_t));
    int rc = ORC_OK;
    if (!acc || !W || !c) {
        rc = ORC_ERR_NOMEM;
        goto done;
    }
    /* as in orc_sparse_average: blocks of parameters, one thread each, and
       inside a block the clients in order */
    const int64_t B = (int64_t)1 << 16;
    const int64_t nb = (len + B - 1) / B;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < nb; ++b) {
        const int64_t lo = first + b * B, hi = lo + B < first + len ? lo + B : first + len;
        for (int k = 0; k < K; ++k) {
            if (n[k] == 0)
                continue;
            for (int64_t j = lower_bound_i64(idx[k], nnz[k], lo); j < nnz[k] && idx[k][j] < hi; ++j) {
                const int64_t i = idx[k][j] - first;
                acc[i] = fmaf((float)n[k], val[k][j], acc[i]);
                W[i] += (uint64_t)n[k];
                c[i] += 1;
            }
        }
    }
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < len; ++i) {
        float r;
        if (W[i] == 0) {
            r = base[i];
        } else {
            const float D = (float)(mode == ORC_DELTAS_ZERO_FILL ? S : W[i]);
            const float q = acc[i] / D;
            r = (mode == ORC_WEIGHTS) ? q : base[i] + q;
        }
        out[i] = r;
        if (count)
            count[i] = c[i];
        if (wsum)
            wsum[i] = W[i];
    }
done:
    free(acc);
    free(W);
    free(c);
    return rc;
}

/*
 * Order-independent checksum of a buffer of elements of the given type:
 * H = sum over i of fmix64(i * 0x9E3779B97F4A7C15 XOR bits_i), modulo
 * 2^64, where bits_i is the element's raw bit pattern (16 or 32 bits) and
 * fmix64 is the 64-bit finalizer of Austin Appleby's MurmurHash3.
 */
static uint64_t fmix64(uint64_t k)
{
    k ^= k >> 33;
    k *= 0xff51afd7ed558ccdULL;
    k ^= k >> 33;
    k *= 0xc4ceb9fe1a85ec53ULL;
    k ^= k >> 33;
    return k;
}

uint64_t orc_checksum(const void *buf, int64_t count, int dtype, int64_t first)
{
    /* `first` is the index of buf[0] in the whole buffer, so the checksum of
       a buffer is the sum of the checksums of its pieces */
    uint64_t h = 0;
#pragma omp parallel for schedule(static) reduction(+ : h) if (count > 65536)
    for (int64_t j = 0; j < count; ++j) {
        uint64_t bits = (dtype == ORC_F32) ? (uint64_t)((const uint32_t *)buf)[j]
                                           : (uint64_t)((const uint16_t *)buf)[j];
        uint64_t i = (uint64_t)(first + j);
        h += fmix64((i * 0x9E3779B97F4A7C15ULL) ^ bits);
    }
    return h;
}

/*
 * Sum of a buffer's element values, a diagnostic that goes with the
 * checksum (no page defines one).  Its definition: the exact real sum of the
 * values, rounded once to the nearest fp64 value (ties to even), so that no
 * order of addition enters.  Every finite fp32 value is an integer multiple
 * of 2^-149 (and a bf16 value is an fp32 value), so the exact sum is an
 * integer number of 2^-149 units; it is held in base-2^32 digits kept in
 * int64 (room for 2^30 additions between carry passes).  Special values
 * follow IEEE addition, whose result does not depend on the order either:
 * a NaN, or infinities of both signs, give NaN; otherwise an infinity gives
 * itself.  A zero sum is +0.
 */
#define SUM_DIGITS 12
static int64_t sum_carry_period = (int64_t)1 << 30;

/* test hook: carry passes more often, to exercise them on small inputs */
void orc_sum_set_carry_period(int64_t p) { sum_carry_period = p > 0 ? p : (int64_t)1 << 30; }

static void sum_carry(int64_t *d)
{
    const int64_t R = (int64_t)1 << 32;
    for (int L = 0; L + 1 < SUM_DIGITS; ++L) {
        int64_t c = d[L] >= 0 ? d[L] / R : -((-d[L] + R - 1) / R); /* floor(d / R) */
        d[L] -= c * R;
        d[L + 1] += c;
    }
}

static int sum_bit(const int64_t *d, int i) { return (int)((d[i / 32] >> (i % 32)) & 1); }

double orc_sum(const void *buf, int64_t count, int dtype)
{
    int64_t d[SUM_DIGITS] = {0};
    int nan = 0, pinf = 0, ninf = 0;
    for (int64_t j = 0; j < count; ++j) {
        uint32_t u = (dtype == ORC_F32) ? ((const uint32_t *)buf)[j]
                                        : (uint32_t)((const uint16_t *)buf)[j] << 16;
        uint32_t e = (u >> 23) & 0xFFu, f = u & 0x7FFFFFu;
        int neg = (int)(u >> 31);
        if (e == 0xFFu) {
            if (f)
                nan = 1;
            else if (neg)
                ninf = 1;
            else
                pinf = 1;
            continue;
        }
        /* value = m * 2^(p - 149) */
        uint64_t m = e ? (f | 0x800000u) : f;
        int p = e ? (int)e - 1 : 0;
        uint64_t v = m << (p % 32);
        int64_t lo = (int64_t)(v & 0xFFFFFFFFu), hi = (int64_t)(v >> 32);
        d[p / 32] += neg ? -lo : lo;
        d[p / 32 + 1] += neg ? -hi : hi;
        if ((j + 1) % sum_carry_period == 0)
            sum_carry(d);
    }
    if (nan || (pinf && ninf))
        return NAN;
    if (pinf)
        return INFINITY;
    if (ninf)
        return -INFINITY;
    sum_carry(d);
    int neg = d[SUM_DIGITS - 1] < 0;
    if (neg) {
        for (int L = 0; L < SUM_DIGITS; ++L)
            d[L] = -d[L];
        sum_carry(d);
    }
    /* magnitude: digits in [0, 2^32); B = its highest set bit */
    int B = 32 * SUM_DIGITS - 1;
    while (B >= 0 && !sum_bit(d, B))
        --B;
    if (B < 0)
        return 0.0;
    uint64_t mant = 0;
    for (int i = 0; i <= 52; ++i)
        if (B - i >= 0 && sum_bit(d, B - i))
            mant |= (uint64_t)1 << (52 - i);
    int round = B - 53 >= 0 ? sum_bit(d, B - 53) : 0;
    int sticky = 0;
    for (int i = 0; i < B - 53; ++i)
        sticky |= sum_bit(d, i);
    if (round && (sticky || (mant & 1u))) {
        mant += 1;
        if (mant == (uint64_t)1 << 53) {
            mant >>= 1;
            B += 1;
        }
    }
    double r = ldexp((double)mant, B - 52 - 149);
    return neg ? -r : r;
}

/*
 * Client-side top-k selection for partial sharing.  A client shares only a
 * fraction of its update, which it chooses itself (Clara page, introduction
 * and client-side workflow section); the fraction kept is the k = floor(p*N)
 * entries of largest magnitude.  Readings where the page is silent: the
 * order is by |value| -- precisely, by the magnitude bit pattern (the value's
 * bits with the sign cleared, of the fp32 value; a bf16 value is widened to
 * fp32 exactly), which orders finite values and infinities by |value| and
 * places NaNs above infinity; -0 and +0 tie; ties go to the lower index.  The
 * result is the k chosen indices in increasing order with their values.
 *
 * Written as the definition: every (key, index) pair sorted by key
 * descending then index ascending, the first k taken, then re-sorted by
 * index.
 */
typedef struct {
    uint32_t key;
    int64_t index;
} orc_rank;

static int by_key_desc_then_index(const void *a, const void *b)
{
    const orc_rank *x = (const orc_rank *)a, *y = (const orc_rank *)b;
    if (x->key != y->key)
        return x->key > y->key ? -1 : 1;
    return (x->index > y->index) - (x->index < y->index);
}

static int by_index(const void *a, const void *b)
{
    int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    return (x > y) - (x < y);
}

static uint32_t magnitude_key(const void *buf, int dtype, int64_t i)
{
    uint32_t bits;
    if (dtype == ORC_F32)
        memcpy(&bits, (const char *)buf + 4 * i, 4);
    else
        bits = (uint32_t)((const uint16_t *)buf)[i] << 16;
    return bits & 0x7FFFFFFFu;
}

int orc_topk(const void *x, int dtype, int64_t N, int64_t k, int64_t *idx_out, float *val_out)
{
    if (!dtype_ok(dtype) || N < 0 || k < 0 || k > N || (N > 0 && !x))
        return ORC_ERR_ARG;
    if (k == 0)
        return ORC_OK;
    orc_rank *r = (orc_rank *)malloc((size_t)N * sizeof *r);
    if (!r)
        return ORC_ERR_NOMEM;
    for (int64_t i = 0; i < N; ++i) {
        r[i].key = magnitude_key(x, dtype, i);
        r[i].index = i;
    }
    qsort(r, (size_t)N, sizeof *r, by_key_desc_then_index);
    for (int64_t j = 0; j < k; ++j)
        idx_out[j] = r[j].index;
    free(r);
    qsort(idx_out, (size_t)k, sizeof *idx_out, by_index);
    for (int64_t j = 0; j < k; ++j)
        val_out[j] = (float)value_at(x, dtype, idx_out[j]);
    return ORC_OK;
}
