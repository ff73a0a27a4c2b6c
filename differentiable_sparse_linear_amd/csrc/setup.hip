// Pattern set-up, once per sla_create.
//
// Validation: row_ptr[0] = 0, non-decreasing, row_ptr[n] = nnz; columns in
// range, strictly ascending per row; the diagonal stored (its position is
// kept in diagpos for the Jacobi preconditioner -- the native backend's only
// preconditioner per the torch-sla explainer's Significance section).
//
// Transpose map (needed by the adjoint solve with A^T, Methodology section 2,
// linear systems): a stable LSD radix sort of (col[k], k) by column gives
// perm[kt] = k in column-major order with rows ascending inside each column,
// so row kt of A^T is sorted; col_t[kt] = row(perm[kt]); row_ptr_t[c] is the
// first kt whose key is >= c, found from the sorted keys without atomics.
//
// Per-row loops over a row's entries serialise on long rows (a graph hub
// of half a million entries), so patterns whose longest row exceeds
// kShortRow are checked entry by entry from the row of every entry.
#include <hipcub/hipcub.hpp>

#include "sla_internal.h"

namespace sla {

template <typename IT>
__global__ __launch_bounds__(kBlock) void check_rowptr_kernel(const IT *__restrict__ rp, int64_t n,
                                                              int64_t nnz, int32_t *flag) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    int bad = 0;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride) {
        const IT a = rp[i], b = rp[i + 1];
        if (b < a) bad = 1;
        if (i == 0 && a != 0) bad = 1;
        if (i == n - 1 && (int64_t)b != nnz) bad = 1;
    }
    raise_flag(bad, flag);
}

template <typename IT>
__global__ __launch_bounds__(kBlock) void check_cols_kernel(const IT *__restrict__ rp,
                                                            const int32_t *__restrict__ col,
                                                            int64_t n, IT *__restrict__ diagpos,
                                                            int32_t *flag) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    int bad = 0;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride) {
        const IT e = rp[i + 1];
        int64_t prev = -1;
        IT dpos = -1;
        for (IT k = rp[i]; k < e; ++k) {
            const int64_t c = col[k];
            if (c < 0 || c >= n || c <= prev) bad = 1;
            if (c == i) dpos = k;
            prev = c;
        }
        if (dpos < 0) bad = 1;
        diagpos[i] = dpos;
    }
    raise_flag(bad, flag);
}

// The row of every entry, first step: each row that holds entries writes
// its index at its first entry (rowidx zeroed before); an inclusive
// max-scan then carries every mark over the row's other entries (an empty
// row writes nothing and its index is below the next row's).
template <typename IT>
__global__ __launch_bounds__(kBlock) void row_start_kernel(const IT *__restrict__ rp, int64_t n,
                                                           int32_t *__restrict__ rowidx) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride)
        if (rp[i + 1] > rp[i]) rowidx[rp[i]] = (int32_t)i;
}

// Entry k of row r = rowidx[k]: its column in range and above the previous
// entry's when that entry is in the same row; the diagonal's position
// (diagpos preset to -1; check_diag_kernel flags the rows without one).
template <typename IT>
__global__ __launch_bounds__(kBlock) void check_cols_entries_kernel(
    const IT *__restrict__ rp, const int32_t *__restrict__ col, const int32_t *__restrict__ rowidx,
    int64_t n, int64_t nnz, IT *__restrict__ diagpos, int32_t *flag) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    int bad = 0;
    for (int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x; k < nnz; k += stride) {
        const int32_t r = rowidx[k];
        const int64_t c = col[k];
        if (c < 0 || c >= n) bad = 1;
        if (k > (int64_t)rp[r] && c <= (int64_t)col[k - 1]) bad = 1;
        if (c == r) diagpos[r] = (IT)k;
    }
    raise_flag(bad, flag);
}

template <typename IT>
__global__ __launch_bounds__(kBlock) void check_diag_kernel(const IT *__restrict__ diagpos,
                                                            int64_t n, int32_t *flag) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    int bad = 0;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride)
        if (diagpos[i] < 0) bad = 1;
    raise_flag(bad, flag);
}

__global__ __launch_bounds__(kBlock) void iota_kernel(int32_t *a, int64_t m) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x; k < m; k += stride)
        a[k] = (int32_t)k;
}

__global__ __launch_bounds__(kBlock) void col_t_kernel(const int32_t *__restrict__ perm,
                                                       const int32_t *__restrict__ rowidx,
                                                       int32_t *__restrict__ col_t, int64_t m) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x; k < m; k += stride)
        col_t[k] = rowidx[perm[k]];
}

// rp_t[c] = first position whose sorted key is >= c, for c in [0, n]
template <typename IT>
__global__ __launch_bounds__(kBlock) void rowptr_t_kernel(const int32_t *__restrict__ keys,
                                                          int64_t m, int64_t n, IT *__restrict__ rp_t) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x; k <= m; k += stride) {
        const int64_t lo = (k == 0) ? -1 : (int64_t)keys[k - 1];
        const int64_t hi = (k == m) ? n : (int64_t)keys[k];
        for (int64_t c = lo + 1; c <= hi; ++c) rp_t[c] = (IT)k;
    }
}

template <typename IT>
__global__ __launch_bounds__(kBlock) void max_row_kernel(const IT *__restrict__ rp, int64_t n,
                                                         int32_t *out) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    int64_t m = 0;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride) {
        const int64_t len = (int64_t)(rp[i + 1] - rp[i]);
        m = len > m ? len : m;
    }
    int32_t mi = m > 0x7fffffff ? 0x7fffffff : (int32_t)m;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const int32_t o = __shfl_xor(mi, off, 64);
        mi = o > mi ? o : mi;
    }
    __shared__ int32_t wm[kWaves];
    if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = mi;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kWaves; ++w) mi = wm[w] > mi ? wm[w] : mi;
        atomicMax(out, mi > wm[0] ? mi : wm[0]);  // one atomic per block
    }
}

// One thread per row: the offsets of the row's columns from its tile's first
// row; any offset outside int16 sets *bad.  `out` may be null (check only).
template <typename IT>
__global__ __launch_bounds__(kBlock) void col16_kernel(const IT *__restrict__ rp,
                                                       const int32_t *__restrict__ col, int64_t n,
                                                       int16_t *__restrict__ out, int32_t *bad) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    int b = 0;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride) {
        const int64_t row0 = i / kTileRows * kTileRows;
        for (IT k = rp[i]; k < rp[i + 1]; ++k) {
            const int64_t d = (int64_t)col[k] - row0;
            const bool ok = d >= -32768 && d <= 32767;
            b |= !ok;
            if (out && ok) out[k] = (int16_t)d;
        }
    }
    raise_flag(b, bad);
}

// The same entry by entry, from the row of every entry.
__global__ __launch_bounds__(kBlock) void col16_entries_kernel(const int32_t *__restrict__ col,
                                                               const int32_t *__restrict__ rowidx,
                                                               int64_t nnz,
                                                               int16_t *__restrict__ out,
                                                               int32_t *bad) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    int b = 0;
    for (int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x; k < nnz; k += stride) {
        const int64_t row0 = (int64_t)rowidx[k] / kTileRows * kTileRows;
        const int64_t d = (int64_t)col[k] - row0;
        const bool ok = d >= -32768 && d <= 32767;
        b |= !ok;
        if (out && ok) out[k] = (int16_t)d;
    }
    raise_flag(b, bad);
}

// Distinct diagonals: each block gathers the offsets (col - row) of its
// rows into a small set in LDS, then merges it into the global set `table`
// [kMaxDiags] (kEmpty = free slot).  Insertion walks the slots in order and
// claims the first free one with compare-and-swap, so no value is stored
// twice; a value finding every slot taken by others sets *over.
constexpr int32_t kEmpty = INT32_MIN;

__device__ __forceinline__ bool set_insert(int32_t *tab, int32_t v) {
    for (int q = 0; q < kMaxDiags; ++q) {
        const int32_t old = atomicCAS(&tab[q], kEmpty, v);
        if (old == kEmpty || old == v) return true;
    }
    return false;
}

template <typename IT>
__global__ __launch_bounds__(kBlock) void diag_collect_kernel(const IT *__restrict__ rp,
                                                              const int32_t *__restrict__ col,
                                                              int64_t n, int32_t *table,
                                                              int32_t *over) {
    __shared__ int32_t loc[kMaxDiags];
    __shared__ int32_t bad;
    if (threadIdx.x < kMaxDiags) loc[threadIdx.x] = kEmpty;
    if (threadIdx.x == 0) bad = 0;
    __syncthreads();
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride)
        for (IT k = rp[i]; k < rp[i + 1]; ++k)
            if (!set_insert(loc, (int32_t)((int64_t)col[k] - i))) bad = 1;
    __syncthreads();
    if (threadIdx.x < kMaxDiags && loc[threadIdx.x] != kEmpty)
        if (!set_insert(table, loc[threadIdx.x])) atomicOr(over, 1);
    if (threadIdx.x == 0 && bad) atomicOr(over, 1);
}

// msk[i] = bit q set for every stored entry of row i on diagonal dlt[q].
template <typename IT>
__global__ __launch_bounds__(kBlock) void diag_mask_kernel(const IT *__restrict__ rp,
                                                           const int32_t *__restrict__ col,
                                                           int64_t n,
                                                           const int32_t *__restrict__ dlt,
                                                           int32_t ndiag,
                                                           uint16_t *__restrict__ msk) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride) {
        uint32_t m = 0;
        for (IT k = rp[i]; k < rp[i + 1]; ++k) {
            const int64_t d = (int64_t)col[k] - i;
            for (int q = 0; q < ndiag; ++q)
                if (dlt[q] == d) m |= 1u << q;
        }
        msk[i] = (uint16_t)m;
    }
}

static unsigned blocks_for(int64_t m) {
    int64_t b = (m + kBlock - 1) / kBlock;
    if (b > 65536) b = 65536;
    if (b < 1) b = 1;
    return (unsigned)b;
}

// rowidx[k] = the row of entry k, for a valid row_ptr (synchronizes the
// stream; temporary scan storage).
template <typename IT>
hipError_t setup_row_index(const IT *rp, int64_t n, int64_t nnz, int32_t *rowidx, hipStream_t s) {
    hipError_t e = hipMemsetAsync(rowidx, 0, sizeof(int32_t) * nnz, s);
    if (e != hipSuccess) return e;
    row_start_kernel<IT><<<blocks_for(n), kBlock, 0, s>>>(rp, n, rowidx);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    size_t tb = 0;
    if ((e = hipcub::DeviceScan::InclusiveScan(nullptr, tb, rowidx, hipcub::Max(), nnz, s)) !=
        hipSuccess)
        return e;
    void *temp = nullptr;
    if ((e = hipMalloc(&temp, tb > 0 ? tb : 1)) != hipSuccess) return e;
    e = hipcub::DeviceScan::InclusiveScan(temp, tb, rowidx, hipcub::Max(), nnz, s);
    const hipError_t es = hipStreamSynchronize(s);
    (void)hipFree(temp);
    return e != hipSuccess ? e : es;
}

// Whether a pattern is checked entry by entry: a row past kShortRow and
// fewer than 2^31 entries (the row of every entry, 4 bytes each, held
// while checking).
inline bool entrywise(int32_t max_len, int64_t nnz) {
    return max_len > kShortRow && nnz < ((int64_t)1 << 31);
}

template <typename IT>
hipError_t setup_validate(const IT *rp, const int32_t *col, int64_t n, int64_t nnz, IT *diagpos,
                          int32_t *flag, hipStream_t s) {
    int32_t h = 0;
    hipError_t e = hipMemsetAsync(flag, 0, sizeof(int32_t), s);
    if (e != hipSuccess) return e;
    check_rowptr_kernel<IT><<<blocks_for(n), kBlock, 0, s>>>(rp, n, nnz, flag);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = hipMemcpyAsync(&h, flag, sizeof(int32_t), hipMemcpyDeviceToHost, s)) != hipSuccess)
        return e;
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;
    if (h) return hipSuccess;  // flag stays set: row_ptr invalid, columns not read
    int32_t max_len = 0;
    if ((e = setup_max_row<IT>(rp, n, flag, &max_len, s)) != hipSuccess) return e;
    if ((e = hipMemsetAsync(flag, 0, sizeof(int32_t), s)) != hipSuccess) return e;
    if (!entrywise(max_len, nnz)) {
        check_cols_kernel<IT><<<blocks_for(n), kBlock, 0, s>>>(rp, col, n, diagpos, flag);
        return hipGetLastError();
    }
    int32_t *rowidx = nullptr;
    if ((e = hipMalloc(&rowidx, sizeof(int32_t) * nnz)) != hipSuccess) return e;
    do {
        if ((e = setup_row_index<IT>(rp, n, nnz, rowidx, s)) != hipSuccess) break;
        if ((e = hipMemsetAsync(diagpos, 0xff, sizeof(IT) * n, s)) != hipSuccess) break;
        check_cols_entries_kernel<IT>
            <<<blocks_for(nnz), kBlock, 0, s>>>(rp, col, rowidx, n, nnz, diagpos, flag);
        check_diag_kernel<IT><<<blocks_for(n), kBlock, 0, s>>>(diagpos, n, flag);
        if ((e = hipGetLastError()) != hipSuccess) break;
        e = hipStreamSynchronize(s);  // rowidx is freed next
    } while (0);
    (void)hipFree(rowidx);
    return e;
}

// Longest row of a valid pattern (synchronizes the stream).
template <typename IT>
hipError_t setup_max_row(const IT *rp, int64_t n, int32_t *scratch, int32_t *out, hipStream_t s) {
    hipError_t e = hipMemsetAsync(scratch, 0, sizeof(int32_t), s);
    if (e != hipSuccess) return e;
    // a few hundred blocks striding over the rows: the atomics on one word
    // serialise, so their number is kept small
    const unsigned nb = blocks_for(n) < 512 ? blocks_for(n) : 512;
    max_row_kernel<IT><<<nb, kBlock, 0, s>>>(rp, n, scratch);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = hipMemcpyAsync(out, scratch, sizeof(int32_t), hipMemcpyDeviceToHost, s)) != hipSuccess)
        return e;
    return hipStreamSynchronize(s);
}

template <typename IT>
hipError_t setup_diag(const IT *rp, const int32_t *col, int64_t n, int32_t *dev_table,
                      int32_t *scratch, int32_t *dlt, int32_t *ndiag, hipStream_t s) {
    *ndiag = 0;
    int32_t init[kMaxDiags];
    for (int q = 0; q < kMaxDiags; ++q) init[q] = kEmpty;
    hipError_t e = hipMemcpyAsync(dev_table, init, sizeof(init), hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return e;
    if ((e = hipMemsetAsync(scratch, 0, sizeof(int32_t), s)) != hipSuccess) return e;
    const unsigned nb = blocks_for(n) < 1024 ? blocks_for(n) : 1024;
    diag_collect_kernel<IT><<<nb, kBlock, 0, s>>>(rp, col, n, dev_table, scratch);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    int32_t tab[kMaxDiags], over = 1;
    if ((e = hipMemcpyAsync(tab, dev_table, sizeof(tab), hipMemcpyDeviceToHost, s)) != hipSuccess)
        return e;
    if ((e = hipMemcpyAsync(&over, scratch, sizeof(int32_t), hipMemcpyDeviceToHost, s)) !=
        hipSuccess)
        return e;
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;  // init, tab: host buffers
    if (over) return hipSuccess;
    int m = 0;
    for (int q = 0; q < kMaxDiags; ++q)
        if (tab[q] != kEmpty) dlt[m++] = tab[q];
    for (int a = 1; a < m; ++a)  // ascending
        for (int b = a; b > 0 && dlt[b - 1] > dlt[b]; --b) {
            const int32_t t = dlt[b];
            dlt[b] = dlt[b - 1];
            dlt[b - 1] = t;
        }
    for (int q = m; q < kMaxDiags; ++q) dlt[q] = 0;
    *ndiag = m;
    return hipSuccess;
}

template <typename IT>
hipError_t setup_diag_masks(const IT *rp, const int32_t *col, int64_t n, const int32_t *dlt_dev,
                            int32_t ndiag, uint16_t *msk, hipStream_t s) {
    diag_mask_kernel<IT><<<blocks_for(n), kBlock, 0, s>>>(rp, col, n, dlt_dev, ndiag, msk);
    return hipGetLastError();
}

template <typename IT>
hipError_t setup_col16(const IT *rp, const int32_t *col, int64_t n, int64_t nnz, int32_t max_len,
                       int16_t *out, int32_t *scratch, int32_t *fits, hipStream_t s) {
    hipError_t e = hipMemsetAsync(scratch, 0, sizeof(int32_t), s);
    if (e != hipSuccess) return e;
    if (!entrywise(max_len, nnz)) {
        col16_kernel<IT><<<blocks_for(n), kBlock, 0, s>>>(rp, col, n, out, scratch);
        e = hipGetLastError();
    } else {
        int32_t *rowidx = nullptr;
        if ((e = hipMalloc(&rowidx, sizeof(int32_t) * nnz)) != hipSuccess) return e;
        e = setup_row_index<IT>(rp, n, nnz, rowidx, s);
        if (e == hipSuccess) {
            col16_entries_kernel<<<blocks_for(nnz), kBlock, 0, s>>>(col, rowidx, nnz, out,
                                                                    scratch);
            e = hipGetLastError();
            const hipError_t es = hipStreamSynchronize(s);  // rowidx is freed next
            if (e == hipSuccess) e = es;
        }
        (void)hipFree(rowidx);
    }
    if (e != hipSuccess) return e;
    int32_t bad = 1;
    if ((e = hipMemcpyAsync(&bad, scratch, sizeof(int32_t), hipMemcpyDeviceToHost, s)) != hipSuccess)
        return e;
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;
    *fits = bad ? 0 : 1;
    return hipSuccess;
}

template <typename IT>
hipError_t setup_transpose(const IT *rp, const int32_t *col, int64_t n, int64_t nnz, IT *rp_t,
                           int32_t *col_t, int32_t *perm, hipStream_t s) {
    int32_t *keys_out = nullptr, *vals_in = nullptr, *rowidx = nullptr;
    void *temp = nullptr;
    size_t temp_bytes = 0;
    int end_bit = 1;
    while (end_bit < 32 && ((int64_t)1 << end_bit) < n) ++end_bit;
    const int m = (int)nnz;
    hipError_t e = hipSuccess;
    do {
        if ((e = hipMalloc(&keys_out, sizeof(int32_t) * nnz)) != hipSuccess) break;
        if ((e = hipMalloc(&vals_in, sizeof(int32_t) * nnz)) != hipSuccess) break;
        if ((e = hipMalloc(&rowidx, sizeof(int32_t) * nnz)) != hipSuccess) break;
        iota_kernel<<<blocks_for(nnz), kBlock, 0, s>>>(vals_in, nnz);
        if ((e = hipGetLastError()) != hipSuccess) break;
        if ((e = setup_row_index<IT>(rp, n, nnz, rowidx, s)) != hipSuccess) break;
        e = hipcub::DeviceRadixSort::SortPairs(nullptr, temp_bytes, col, keys_out, vals_in, perm,
                                               m, 0, end_bit, s);
        if (e != hipSuccess) break;
        if ((e = hipMalloc(&temp, temp_bytes > 0 ? temp_bytes : 1)) != hipSuccess) break;
        e = hipcub::DeviceRadixSort::SortPairs(temp, temp_bytes, col, keys_out, vals_in, perm, m,
                                               0, end_bit, s);
        if (e != hipSuccess) break;
        col_t_kernel<<<blocks_for(nnz), kBlock, 0, s>>>(perm, rowidx, col_t, nnz);
        rowptr_t_kernel<IT><<<blocks_for(nnz + 1), kBlock, 0, s>>>(keys_out, nnz, n, rp_t);
        if ((e = hipGetLastError()) != hipSuccess) break;
        e = hipStreamSynchronize(s);
    } while (0);
    (void)hipFree(keys_out);
    (void)hipFree(vals_in);
    (void)hipFree(rowidx);
    (void)hipFree(temp);
    return e;
}

// Launchers of the single checks, for callers that keep their own flags
// (each raises *flag or atomically maxes *out, which must start at 0); they
// allocate nothing and do not synchronize.
template <typename IT>
hipError_t launch_check_rowptr(const IT *rp, int64_t n, int64_t nnz, int32_t *flag,
                               hipStream_t s) {
    check_rowptr_kernel<IT><<<blocks_for(n), kBlock, 0, s>>>(rp, n, nnz, flag);
    return hipGetLastError();
}

template <typename IT>
hipError_t launch_check_cols_rows(const IT *rp, const int32_t *col, int64_t n, IT *diagpos,
                                  int32_t *flag, hipStream_t s) {
    check_cols_kernel<IT><<<blocks_for(n), kBlock, 0, s>>>(rp, col, n, diagpos, flag);
    return hipGetLastError();
}

template <typename IT>
hipError_t launch_max_row(const IT *rp, int64_t n, int32_t *out, hipStream_t s) {
    const unsigned nb = blocks_for(n) < 512 ? blocks_for(n) : 512;
    max_row_kernel<IT><<<nb, kBlock, 0, s>>>(rp, n, out);
    return hipGetLastError();
}

#define SLA_CHECK_INST(IT)                                                                     \
    template hipError_t launch_check_rowptr<IT>(const IT *, int64_t, int64_t, int32_t *,       \
                                                hipStream_t);                                  \
    template hipError_t launch_check_cols_rows<IT>(const IT *, const int32_t *, int64_t, IT *, \
                                                   int32_t *, hipStream_t);                    \
    template hipError_t launch_max_row<IT>(const IT *, int64_t, int32_t *, hipStream_t);
SLA_CHECK_INST(int32_t)
SLA_CHECK_INST(int64_t)
#undef SLA_CHECK_INST

template hipError_t setup_validate<int32_t>(const int32_t *, const int32_t *, int64_t, int64_t,
                                            int32_t *, int32_t *, hipStream_t);
template hipError_t setup_validate<int64_t>(const int64_t *, const int32_t *, int64_t, int64_t,
                                            int64_t *, int32_t *, hipStream_t);
template hipError_t setup_diag<int32_t>(const int32_t *, const int32_t *, int64_t, int32_t *,
                                        int32_t *, int32_t *, int32_t *, hipStream_t);
template hipError_t setup_diag<int64_t>(const int64_t *, const int32_t *, int64_t, int32_t *,
                                        int32_t *, int32_t *, int32_t *, hipStream_t);
template hipError_t setup_diag_masks<int32_t>(const int32_t *, const int32_t *, int64_t,
                                              const int32_t *, int32_t, uint16_t *, hipStream_t);
template hipError_t setup_diag_masks<int64_t>(const int64_t *, const int32_t *, int64_t,
                                              const int32_t *, int32_t, uint16_t *, hipStream_t);
template hipError_t setup_col16<int32_t>(const int32_t *, const int32_t *, int64_t, int64_t,
                                         int32_t, int16_t *, int32_t *, int32_t *, hipStream_t);
template hipError_t setup_col16<int64_t>(const int64_t *, const int32_t *, int64_t, int64_t,
                                         int32_t, int16_t *, int32_t *, int32_t *, hipStream_t);
template hipError_t setup_max_row<int32_t>(const int32_t *, int64_t, int32_t *, int32_t *,
                                           hipStream_t);
template hipError_t setup_max_row<int64_t>(const int64_t *, int64_t, int32_t *, int32_t *,
                                           hipStream_t);
template hipError_t setup_transpose<int32_t>(const int32_t *, const int32_t *, int64_t, int64_t,
                                             int32_t *, int32_t *, int32_t *, hipStream_t);
template hipError_t setup_transpose<int64_t>(const int64_t *, const int32_t *, int64_t, int64_t,
                                             int64_t *, int32_t *, int32_t *, hipStream_t);

}  // namespace sla
