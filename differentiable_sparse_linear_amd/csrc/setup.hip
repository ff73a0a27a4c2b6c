// Pattern set-up, once per sla_create.
//
// Validation: row_ptr[0] = 0, non-decreasing, row_ptr[n] = nnz; columns in
// range, strictly ascending per row; the diagonal stored (its position is
// kept in diagpos for the Jacobi preconditioner -- the native backend's only
// preconditioner per the torch-sla explainer's Significance section).
//
// Row of every entry (rowidx): each row that holds entries marks its first
// entry with its index, and an inclusive max-scan carries every mark over
// the row's other entries.
//
// Transpose map (needed by the adjoint solve with A^T, Methodology section 2,
// linear systems): a stable least-significant-digit radix sort of the pairs
// (col[k], k) by column, eight bits per pass.  Each pass counts the digits
// of every tile of entries (a histogram in LDS), turns the counts, ordered
// digit by digit and tile by tile, into starting positions by an exclusive
// scan, and scatters each tile's entries in their original order: within a
// round of 256 entries each wavefront finds the lanes that share a lane's
// digit with eight ballots, one per digit bit, and takes the lane's rank
// among them; counters in LDS carry the ranks over the wavefronts and the
// rounds.  Entries of equal digit therefore keep their order, so after the
// last pass perm[kt] = k lists the entries column by column with rows
// ascending inside each column, and row kt of A^T is sorted; col_t[kt] =
// row(perm[kt]); row_ptr_t[c] is the first kt whose key is >= c, found from
// the sorted keys.  The scans are a reduce-then-scan over tiles: per-tile
// totals, one workgroup scanning the totals, then each tile scanned with
// its carry.
//
// Per-row loops over a row's entries serialise on long rows (a graph hub
// of half a million entries), so patterns whose longest row exceeds
// kShortRow are checked entry by entry from the row of every entry.
//
// Temporaries (the row of every entry, the sort's keys and values, digit
// counts, scan totals) live in one allocation that sla_create makes for the
// set-up and releases at its end (SetupScratch).
#include "sla_internal.h"

namespace sla {

// Threads per workgroup of every set-up kernel (independent of the solver
// kernels' block size).
constexpr int kSetupThreads = 256;

template <typename IT>
__global__ __launch_bounds__(kSetupThreads) void check_rowptr_kernel(const IT *__restrict__ rp, int64_t n,
                                                              int64_t nnz, int32_t *flag) {
    const int64_t stride = (int64_t)gridDim.x * kSetupThreads;
    int bad = 0;
    for (int64_t i = (int64_t)blockIdx.x * kSetupThreads + threadIdx.x; i < n; i += stride) {
        const IT a = rp[i], b = rp[i + 1];
        if (b < a) bad = 1;
        if (i == 0 && a != 0) bad = 1;
        if (i == n - 1 && (int64_t)b != nnz) bad = 1;
    }
    raise_flag(bad, flag);
}

template <typename IT>
__global__ __launch_bounds__(kSetupThreads) void check_cols_kernel(const IT *__restrict__ rp,
                                                            const int32_t *__restrict__ col,
                                                            int64_t n, IT *__restrict__ diagpos,
                                                            int32_t *flag) {
    const int64_t stride = (int64_t)gridDim.x * kSetupThreads;
    int bad = 0;
    for (int64_t i = (int64_t)blockIdx.x * kSetupThreads + threadIdx.x; i < n; i += stride) {
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
__global__ __launch_bounds__(kSetupThreads) void row_start_kernel(const IT *__restrict__ rp, int64_t n,
                                                           int32_t *__restrict__ rowidx) {
    const int64_t stride = (int64_t)gridDim.x * kSetupThreads;
    for (int64_t i = (int64_t)blockIdx.x * kSetupThreads + threadIdx.x; i < n; i += stride)
        if (rp[i + 1] > rp[i]) rowidx[rp[i]] = (int32_t)i;
}

// Entry k of row r = rowidx[k]: its column in range and above the previous
// entry's when that entry is in the same row; the diagonal's position
// (diagpos preset to -1; check_diag_kernel flags the rows without one).
template <typename IT>
__global__ __launch_bounds__(kSetupThreads) void check_cols_entries_kernel(
    const IT *__restrict__ rp, const int32_t *__restrict__ col, const int32_t *__restrict__ rowidx,
    int64_t n, int64_t nnz, IT *__restrict__ diagpos, int32_t *flag) {
    const int64_t stride = (int64_t)gridDim.x * kSetupThreads;
    int bad = 0;
    for (int64_t k = (int64_t)blockIdx.x * kSetupThreads + threadIdx.x; k < nnz; k += stride) {
        const int32_t r = rowidx[k];
        const int64_t c = col[k];
        if (c < 0 || c >= n) bad = 1;
        if (k > (int64_t)rp[r] && c <= (int64_t)col[k - 1]) bad = 1;
        if (c == r) diagpos[r] = (IT)k;
    }
    raise_flag(bad, flag);
}

template <typename IT>
__global__ __launch_bounds__(kSetupThreads) void check_diag_kernel(const IT *__restrict__ diagpos,
                                                            int64_t n, int32_t *flag) {
    const int64_t stride = (int64_t)gridDim.x * kSetupThreads;
    int bad = 0;
    for (int64_t i = (int64_t)blockIdx.x * kSetupThreads + threadIdx.x; i < n; i += stride)
        if (diagpos[i] < 0) bad = 1;
    raise_flag(bad, flag);
}

// col_t[k] = the row of A entry perm[k] and pinv[perm[k]] = k, the inverse
// map (-1 in col_t for a position outside [0, m), which only a faulty sort
// could leave, so that it shows in the map instead of reading or writing out
// of bounds)
__global__ __launch_bounds__(kSetupThreads) void col_t_kernel(const int32_t *__restrict__ perm,
                                                       const int32_t *__restrict__ rowidx,
                                                       int32_t *__restrict__ col_t,
                                                       int32_t *__restrict__ pinv, int64_t m) {
    const int64_t stride = (int64_t)gridDim.x * kSetupThreads;
    for (int64_t k = (int64_t)blockIdx.x * kSetupThreads + threadIdx.x; k < m; k += stride) {
        const int64_t j = perm[k];
        const bool ok = j >= 0 && j < m;
        col_t[k] = ok ? rowidx[j] : -1;
        if (ok) pinv[j] = (int32_t)k;
    }
}

// rp_t[c] = first position whose sorted key is >= c, for c in [0, n] (keys
// are columns, in [0, n); the loop bounds are clamped to that range all the
// same)
template <typename IT>
__global__ __launch_bounds__(kSetupThreads) void rowptr_t_kernel(const int32_t *__restrict__ keys,
                                                          int64_t m, int64_t n, IT *__restrict__ rp_t) {
    const int64_t stride = (int64_t)gridDim.x * kSetupThreads;
    for (int64_t k = (int64_t)blockIdx.x * kSetupThreads + threadIdx.x; k <= m; k += stride) {
        int64_t lo = (k == 0) ? -1 : (int64_t)keys[k - 1];
        int64_t hi = (k == m) ? n : (int64_t)keys[k];
        lo = lo < -1 ? -1 : lo;
        hi = hi > n ? n : hi;
        for (int64_t c = lo + 1; c <= hi; ++c) rp_t[c] = (IT)k;
    }
}

template <typename IT>
__global__ __launch_bounds__(kSetupThreads) void max_row_kernel(const IT *__restrict__ rp, int64_t n,
                                                         int32_t *out) {
    const int64_t stride = (int64_t)gridDim.x * kSetupThreads;
    int64_t m = 0;
    for (int64_t i = (int64_t)blockIdx.x * kSetupThreads + threadIdx.x; i < n; i += stride) {
        const int64_t len = (int64_t)(rp[i + 1] - rp[i]);
        m = len > m ? len : m;
    }
    int32_t mi = m > 0x7fffffff ? 0x7fffffff : (int32_t)m;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const int32_t o = __shfl_xor(mi, off, 64);
        mi = o > mi ? o : mi;
    }
    __shared__ int32_t wm[kSetupThreads / 64];
    if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = mi;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kSetupThreads / 64; ++w) mi = wm[w] > mi ? wm[w] : mi;
        atomicMax(out, mi > wm[0] ? mi : wm[0]);  // one atomic per block
    }
}

// One thread per row: the offsets of the row's columns from its tile's first
// row; any offset outside int16 sets *bad.  `out` may be null (check only).
template <typename IT>
__global__ __launch_bounds__(kSetupThreads) void col16_kernel(const IT *__restrict__ rp,
                                                       const int32_t *__restrict__ col, int64_t n,
                                                       int16_t *__restrict__ out, int32_t *bad) {
    const int64_t stride = (int64_t)gridDim.x * kSetupThreads;
    int b = 0;
    for (int64_t i = (int64_t)blockIdx.x * kSetupThreads + threadIdx.x; i < n; i += stride) {
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
__global__ __launch_bounds__(kSetupThreads) void col16_entries_kernel(const int32_t *__restrict__ col,
                                                               const int32_t *__restrict__ rowidx,
                                                               int64_t nnz,
                                                               int16_t *__restrict__ out,
                                                               int32_t *bad) {
    const int64_t stride = (int64_t)gridDim.x * kSetupThreads;
    int b = 0;
    for (int64_t k = (int64_t)blockIdx.x * kSetupThreads + threadIdx.x; k < nnz; k += stride) {
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
__global__ __launch_bounds__(kSetupThreads) void diag_collect_kernel(const IT *__restrict__ rp,
                                                              const int32_t *__restrict__ col,
                                                              int64_t n, int32_t *table,
                                                              int32_t *over) {
    __shared__ int32_t loc[kMaxDiags];
    __shared__ int32_t bad;
    if (threadIdx.x < kMaxDiags) loc[threadIdx.x] = kEmpty;
    if (threadIdx.x == 0) bad = 0;
    __syncthreads();
    const int64_t stride = (int64_t)gridDim.x * kSetupThreads;
    for (int64_t i = (int64_t)blockIdx.x * kSetupThreads + threadIdx.x; i < n; i += stride)
        for (IT k = rp[i]; k < rp[i + 1]; ++k)
            if (!set_insert(loc, (int32_t)((int64_t)col[k] - i))) bad = 1;
    __syncthreads();
    if (threadIdx.x < kMaxDiags && loc[threadIdx.x] != kEmpty)
        if (!set_insert(table, loc[threadIdx.x])) atomicOr(over, 1);
    if (threadIdx.x == 0 && bad) atomicOr(over, 1);
}

// msk[i] = bit q set for every stored entry of row i on diagonal dlt[q].
template <typename IT>
__global__ __launch_bounds__(kSetupThreads) void diag_mask_kernel(const IT *__restrict__ rp,
                                                           const int32_t *__restrict__ col,
                                                           int64_t n,
                                                           const int32_t *__restrict__ dlt,
                                                           int32_t ndiag,
                                                           uint16_t *__restrict__ msk) {
    const int64_t stride = (int64_t)gridDim.x * kSetupThreads;
    for (int64_t i = (int64_t)blockIdx.x * kSetupThreads + threadIdx.x; i < n; i += stride) {
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
    int64_t b = (m + kSetupThreads - 1) / kSetupThreads;
    if (b > 65536) b = 65536;
    if (b < 1) b = 1;
    return (unsigned)b;
}

// ------------------------------------------------------------------ scans
//
// Reduce-then-scan of int32 values over tiles of kScanTile, with the sum
// (MAX = false) or the maximum (MAX = true); every value is >= 0, so 0 is
// the identity of both.  A tile is loaded coalesced (element j * kSetupThreads + t
// by thread t) into LDS and read back blocked (thread t owns the kScanItems
// consecutive elements t * kScanItems ...; a padding word after every 16
// keeps those reads off a single bank), scanned in registers and across the
// block, and written back the same way.
constexpr int kScanItems = 16;
constexpr int kScanTile = kSetupThreads * kScanItems;
constexpr int kScanLds = kScanTile + kScanTile / 16;

template <bool MAX>
__device__ __forceinline__ int32_t scan_op(int32_t a, int32_t b) {
    return MAX ? (a > b ? a : b) : a + b;
}

__device__ __forceinline__ int lds_pad(int e) { return e + (e >> 4); }

// Exclusive scan over the block of one value per thread (identity 0);
// *total gets the block's aggregate.  Every thread gets the same total.
template <bool MAX>
__device__ __forceinline__ int32_t block_exclusive(int32_t v, int32_t *total) {
    __shared__ int32_t wsum[kSetupThreads / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int32_t inc = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t u = __shfl_up(inc, off, 64);
        if (lane >= off) inc = scan_op<MAX>(inc, u);
    }
    int32_t exc = __shfl_up(inc, 1, 64);
    if (lane == 0) exc = 0;
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    int32_t carry = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kSetupThreads / 64; ++w) {
        if (w < wave) carry = scan_op<MAX>(carry, wsum[w]);
        all = scan_op<MAX>(all, wsum[w]);
    }
    __syncthreads();  // wsum is reused by the next call
    *total = all;
    return scan_op<MAX>(carry, exc);
}

// Tile b of in[0..m), blocked: thread t gets elements t * kScanItems + j
// (0 past the end).
__device__ __forceinline__ void tile_load(const int32_t *__restrict__ in, int64_t m,
                                          int32_t *sh, int32_t (&v)[kScanItems]) {
    const int64_t base = (int64_t)blockIdx.x * kScanTile;
#pragma unroll
    for (int j = 0; j < kScanItems; ++j) {
        const int e = j * kSetupThreads + threadIdx.x;
        sh[lds_pad(e)] = base + e < m ? in[base + e] : 0;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kScanItems; ++j) v[j] = sh[lds_pad(threadIdx.x * kScanItems + j)];
    __syncthreads();
}

// tot[b] = the aggregate of tile b.
template <bool MAX>
__global__ __launch_bounds__(kSetupThreads) void tile_total_kernel(const int32_t *__restrict__ in,
                                                            int64_t m, int32_t *__restrict__ tot) {
    __shared__ int32_t sh[kScanLds];
    int32_t v[kScanItems];
    tile_load(in, m, sh, v);
    int32_t a = 0;
#pragma unroll
    for (int j = 0; j < kScanItems; ++j) a = scan_op<MAX>(a, v[j]);
    int32_t all;
    block_exclusive<MAX>(a, &all);
    if (threadIdx.x == 0) tot[blockIdx.x] = all;
}

// tot[0..nt) becomes its exclusive scan: one workgroup, kSetupThreads at a time.
template <bool MAX>
__global__ __launch_bounds__(kSetupThreads) void totals_scan_kernel(int32_t *__restrict__ tot,
                                                             int64_t nt) {
    int32_t carry = 0;
    for (int64_t c = 0; c < nt; c += kSetupThreads) {
        const int64_t i = c + threadIdx.x;
        const int32_t v = i < nt ? tot[i] : 0;
        int32_t all;
        const int32_t exc = block_exclusive<MAX>(v, &all);
        if (i < nt) tot[i] = scan_op<MAX>(carry, exc);
        carry = scan_op<MAX>(carry, all);
    }
}

// out = the inclusive (EXCL = false) or exclusive scan of in, tile b
// starting from the exclusive scan of the tile totals, carry[b].  in and
// out may be the same array (each tile is read before it is written).
template <bool MAX, bool EXCL>
__global__ __launch_bounds__(kSetupThreads) void tile_scan_kernel(const int32_t *in, int64_t m,
                                                           const int32_t *__restrict__ carry,
                                                           int32_t *out) {
    __shared__ int32_t sh[kScanLds];
    int32_t v[kScanItems];
    tile_load(in, m, sh, v);
    int32_t a = 0;
#pragma unroll
    for (int j = 0; j < kScanItems; ++j) a = scan_op<MAX>(a, v[j]);
    int32_t all;
    int32_t run = scan_op<MAX>(carry[blockIdx.x], block_exclusive<MAX>(a, &all));
#pragma unroll
    for (int j = 0; j < kScanItems; ++j) {
        const int32_t nx = scan_op<MAX>(run, v[j]);
        sh[lds_pad(threadIdx.x * kScanItems + j)] = EXCL ? run : nx;
        run = nx;
    }
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kScanTile;
#pragma unroll
    for (int j = 0; j < kScanItems; ++j) {
        const int e = j * kSetupThreads + threadIdx.x;
        if (base + e < m) out[base + e] = sh[lds_pad(e)];
    }
}

inline int64_t scan_tiles(int64_t m) { return (m + kScanTile - 1) / kScanTile; }

// data[0..m) becomes its scan in place; tot holds scan_tiles(m) values.
template <bool MAX, bool EXCL>
hipError_t scan_inplace(int32_t *data, int64_t m, int32_t *tot, hipStream_t s) {
    const int64_t nt = scan_tiles(m);
    if (nt < 1) return hipSuccess;
    tile_total_kernel<MAX><<<(unsigned)nt, kSetupThreads, 0, s>>>(data, m, tot);
    totals_scan_kernel<MAX><<<1, kSetupThreads, 0, s>>>(tot, nt);
    tile_scan_kernel<MAX, EXCL><<<(unsigned)nt, kSetupThreads, 0, s>>>(data, m, tot, data);
    return hipGetLastError();
}

// ------------------------------------------------------------------ radix sort
//
// One pass sorts (key, value) pairs stably by the eight bits of the key at
// `shift`.  Tile b is entries [b * kSortTile, (b + 1) * kSortTile), taken in
// kSortRounds rounds of kSetupThreads consecutive entries, wavefront w holding
// entries [r * kSetupThreads + 64 w, r * kSetupThreads + 64 w + 64) of round r.
constexpr int kSortRounds = 16;
constexpr int kSortTile = kSetupThreads * kSortRounds;
constexpr int kRadix = 256;
static_assert(kSetupThreads == kRadix, "one thread per digit in the sort's bookkeeping");
constexpr int kSetupWaves = kSetupThreads / 64;

inline int64_t sort_tiles(int64_t m) { return (m + kSortTile - 1) / kSortTile; }

__device__ __forceinline__ int32_t sort_value(const int32_t *vin, int64_t e) {
    return vin ? vin[e] : (int32_t)e;  // the first pass's value is the entry's index
}

// hist[d * ntiles + b] = entries of tile b whose digit is d.
__global__ __launch_bounds__(kSetupThreads) void digit_count_kernel(const int32_t *__restrict__ key,
                                                             int64_t m, int shift,
                                                             int32_t *__restrict__ hist) {
    __shared__ int32_t h[kRadix];
    h[threadIdx.x] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kSortTile;
    for (int r = 0; r < kSortRounds; ++r) {
        const int64_t e = base + r * kSetupThreads + threadIdx.x;
        if (e < m) atomicAdd(&h[(key[e] >> shift) & (kRadix - 1)], 1);
    }
    __syncthreads();
    hist[(int64_t)threadIdx.x * gridDim.x + blockIdx.x] = h[threadIdx.x];
}

// Stable scatter of tile b: start[d * ntiles + b] is the position of the
// tile's first entry of digit d (the exclusive scan of hist).
__global__ __launch_bounds__(kSetupThreads) void digit_scatter_kernel(
    const int32_t *__restrict__ kin, const int32_t *__restrict__ vin, int64_t m, int shift,
    const int32_t *__restrict__ start, int32_t *__restrict__ kout, int32_t *__restrict__ vout) {
    __shared__ int32_t pos0[kRadix];          // next position of digit d in this tile
    __shared__ int32_t cnt[kSetupWaves][kRadix];   // this round's count of digit d per wavefront
    const int tid = threadIdx.x, wave = tid >> 6;
    pos0[tid] = start[(int64_t)tid * gridDim.x + blockIdx.x];
#pragma unroll
    for (int w = 0; w < kSetupWaves; ++w) cnt[w][tid] = 0;
    __syncthreads();
    const uint64_t below = __lanemask_lt();
    const int64_t base = (int64_t)blockIdx.x * kSortTile;
    for (int r = 0; r < kSortRounds; ++r) {
        const int64_t e = base + r * kSetupThreads + tid;
        const bool act = e < m;
        const int32_t k = act ? kin[e] : 0;
        const int32_t v = act ? sort_value(vin, e) : 0;
        const int d = (k >> shift) & (kRadix - 1);
        // the lanes holding the same digit: agree on all eight bits
        uint64_t peers = __ballot(act);
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
            const bool one = (d >> bit) & 1;
            const uint64_t b1 = __ballot(act && one);
            peers &= one ? b1 : ~b1;
        }
        const int rank = __popcll(peers & below);
        if (act && rank == 0) cnt[wave][d] = __popcll(peers);
        __syncthreads();
        if (act) {
            int32_t p = pos0[d] + rank;
            for (int w = 0; w < wave; ++w) p += cnt[w][d];
            if (p >= 0 && p < m) {
                kout[p] = k;
                vout[p] = v;
            }
        }
        __syncthreads();
        int32_t add = 0;
#pragma unroll
        for (int w = 0; w < kSetupWaves; ++w) {
            add += cnt[w][tid];
            cnt[w][tid] = 0;
        }
        pos0[tid] += add;
        __syncthreads();
    }
}

// ------------------------------------------------------------------ scratch

int64_t setup_scratch_bytes(int64_t nnz, bool rowidx, bool transpose) {
    auto al = [](int64_t b) { return (b + 255) / 256 * 256; };
    int64_t b = 0;
    int64_t scan_len = 0;
    if (rowidx || transpose) {
        b += al(4 * nnz);  // rowidx
        scan_len = nnz;
    }
    if (transpose) {
        const int64_t hist = (int64_t)kRadix * sort_tiles(nnz);
        b += 3 * al(4 * nnz) + al(4 * hist);  // keys x 2, values, digit counts
        scan_len = scan_len > hist ? scan_len : hist;
    }
    if (scan_len) b += al(4 * (scan_tiles(scan_len) + 1));
    return b;
}

void setup_scratch_carve(void *base, int64_t nnz, bool rowidx, bool transpose,
                         SetupScratch *out) {
    auto al = [](int64_t b) { return (b + 255) / 256 * 256; };
    *out = SetupScratch();
    char *p = static_cast<char *>(base);
    int64_t scan_len = 0;
    if (rowidx || transpose) {
        out->rowidx = reinterpret_cast<int32_t *>(p);
        p += al(4 * nnz);
        scan_len = nnz;
    }
    if (transpose) {
        const int64_t hist = (int64_t)kRadix * sort_tiles(nnz);
        out->keys[0] = reinterpret_cast<int32_t *>(p);
        p += al(4 * nnz);
        out->keys[1] = reinterpret_cast<int32_t *>(p);
        p += al(4 * nnz);
        out->vals = reinterpret_cast<int32_t *>(p);
        p += al(4 * nnz);
        out->hist = reinterpret_cast<int32_t *>(p);
        p += al(4 * hist);
        scan_len = scan_len > hist ? scan_len : hist;
    }
    if (scan_len) out->tot = reinterpret_cast<int32_t *>(p);
}

// ------------------------------------------------------------------ set-up steps

// Whether a pattern is checked entry by entry: a row past kShortRow and
// fewer than 2^31 entries (the row of every entry, 4 bytes each, held
// while checking).
bool setup_entrywise(int32_t max_len, int64_t nnz) {
    return max_len > kShortRow && nnz < ((int64_t)1 << 31);
}

template <typename IT>
hipError_t setup_check_rowptr(const IT *rp, int64_t n, int64_t nnz, int32_t *flag, int32_t *bad,
                              hipStream_t s) {
    hipError_t e = hipMemsetAsync(flag, 0, sizeof(int32_t), s);
    if (e != hipSuccess) return e;
    check_rowptr_kernel<IT><<<blocks_for(n), kSetupThreads, 0, s>>>(rp, n, nnz, flag);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = hipMemcpyAsync(bad, flag, sizeof(int32_t), hipMemcpyDeviceToHost, s)) != hipSuccess)
        return e;
    return hipStreamSynchronize(s);
}

// rowidx[k] = the row of entry k, for a valid row_ptr (tot: scan totals).
template <typename IT>
hipError_t setup_row_index(const IT *rp, int64_t n, int64_t nnz, int32_t *rowidx, int32_t *tot,
                           hipStream_t s) {
    hipError_t e = hipMemsetAsync(rowidx, 0, sizeof(int32_t) * nnz, s);
    if (e != hipSuccess) return e;
    row_start_kernel<IT><<<blocks_for(n), kSetupThreads, 0, s>>>(rp, n, rowidx);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return scan_inplace<true, false>(rowidx, nnz, tot, s);
}

// Columns and diagonals of a pattern whose row pointers passed the check
// (synchronizes the stream): per row, or entry by entry from rowidx (not
// null) for patterns with long rows.
template <typename IT>
hipError_t setup_check_cols(const IT *rp, const int32_t *col, int64_t n, int64_t nnz,
                            const int32_t *rowidx, IT *diagpos, int32_t *flag, int32_t *bad,
                            hipStream_t s) {
    hipError_t e = hipMemsetAsync(flag, 0, sizeof(int32_t), s);
    if (e != hipSuccess) return e;
    if (!rowidx) {
        check_cols_kernel<IT><<<blocks_for(n), kSetupThreads, 0, s>>>(rp, col, n, diagpos, flag);
    } else {
        if ((e = hipMemsetAsync(diagpos, 0xff, sizeof(IT) * n, s)) != hipSuccess) return e;
        check_cols_entries_kernel<IT>
            <<<blocks_for(nnz), kSetupThreads, 0, s>>>(rp, col, rowidx, n, nnz, diagpos, flag);
        check_diag_kernel<IT><<<blocks_for(n), kSetupThreads, 0, s>>>(diagpos, n, flag);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = hipMemcpyAsync(bad, flag, sizeof(int32_t), hipMemcpyDeviceToHost, s)) != hipSuccess)
        return e;
    return hipStreamSynchronize(s);
}

// Longest row of a valid pattern (synchronizes the stream).
template <typename IT>
hipError_t setup_max_row(const IT *rp, int64_t n, int32_t *scratch, int32_t *out, hipStream_t s) {
    hipError_t e = hipMemsetAsync(scratch, 0, sizeof(int32_t), s);
    if (e != hipSuccess) return e;
    // a few hundred blocks striding over the rows: the atomics on one word
    // serialise, so their number is kept small
    const unsigned nb = blocks_for(n) < 512 ? blocks_for(n) : 512;
    max_row_kernel<IT><<<nb, kSetupThreads, 0, s>>>(rp, n, scratch);
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
    diag_collect_kernel<IT><<<nb, kSetupThreads, 0, s>>>(rp, col, n, dev_table, scratch);
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
    diag_mask_kernel<IT><<<blocks_for(n), kSetupThreads, 0, s>>>(rp, col, n, dlt_dev, ndiag, msk);
    return hipGetLastError();
}

template <typename IT>
hipError_t setup_col16(const IT *rp, const int32_t *col, int64_t n, int64_t nnz,
                       const int32_t *rowidx, int16_t *out, int32_t *scratch, int32_t *fits,
                       hipStream_t s) {
    hipError_t e = hipMemsetAsync(scratch, 0, sizeof(int32_t), s);
    if (e != hipSuccess) return e;
    if (!rowidx)
        col16_kernel<IT><<<blocks_for(n), kSetupThreads, 0, s>>>(rp, col, n, out, scratch);
    else
        col16_entries_kernel<<<blocks_for(nnz), kSetupThreads, 0, s>>>(col, rowidx, nnz, out, scratch);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    int32_t bad = 1;
    if ((e = hipMemcpyAsync(&bad, scratch, sizeof(int32_t), hipMemcpyDeviceToHost, s)) != hipSuccess)
        return e;
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;
    *fits = bad ? 0 : 1;
    return hipSuccess;
}

template <typename IT>
hipError_t setup_transpose(const IT *rp, const int32_t *col, int64_t n, int64_t nnz, IT *rp_t,
                           int32_t *col_t, int32_t *perm, int32_t *pinv, SetupScratch &scr,
                           hipStream_t s) {
    (void)rp;
    int bits = 1;
    while (bits < 31 && ((int64_t)1 << bits) < n) ++bits;
    const int passes = (bits + 7) / 8;
    const int64_t nt = sort_tiles(nnz);
    const int64_t nh = (int64_t)kRadix * nt;
    hipError_t e = hipSuccess;
    // pass i reads what pass i - 1 wrote; the last pass writes its keys to
    // keys[1] and its values to perm
    const int32_t *kin = col, *vin = nullptr;
    for (int i = 0; i < passes; ++i) {
        const bool last = ((passes - 1 - i) & 1) == 0;
        int32_t *kout = last ? scr.keys[1] : scr.keys[0];
        int32_t *vout = last ? perm : scr.vals;
        digit_count_kernel<<<(unsigned)nt, kSetupThreads, 0, s>>>(kin, nnz, 8 * i, scr.hist);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = scan_inplace<false, true>(scr.hist, nh, scr.tot, s)) != hipSuccess) return e;
        digit_scatter_kernel<<<(unsigned)nt, kSetupThreads, 0, s>>>(kin, vin, nnz, 8 * i, scr.hist,
                                                            kout, vout);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        kin = kout;
        vin = vout;
    }
    // keys[1] holds the sorted columns: the row of every entry of A^T
    scr.rowidx_t = scr.keys[1];
    rowptr_t_kernel<IT><<<blocks_for(nnz + 1), kSetupThreads, 0, s>>>(scr.rowidx_t, nnz, n, rp_t);
    col_t_kernel<<<blocks_for(nnz), kSetupThreads, 0, s>>>(perm, scr.rowidx, col_t, pinv, nnz);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return hipStreamSynchronize(s);
}

// Write positions of the two-pass A^T products (sla_ctx::bpos, lidx).  The
// terms pass walks A's entries in order and stores entry k's term at
// bpos[k]; the row sums then add A^T's rows tile by tile (kTileRows rows of
// A^T).  With bpos = pinv every term is an 8-byte write to a scattered place
// and a cache line of A^T's order is completed by many writes far apart in
// time.  Instead, for each run of A^T's entries that the row sums stage in
// LDS -- a tile of at most kCap entries outside A^T's row plan, or a short
// block of the plan -- the run's entries are kept in A's entry order:
// bpos[k] = the run's first A^T position + the rank of k among the run's
// entries, and lidx at that position = the entry's offset in A^T's order
// inside the run, so that the row sums put every term back in A^T's order in
// LDS before adding.  Since each XCD walks a contiguous range of A's entries
// (the tiles by xcd_tiles, the plan's items likewise), its writes to a run
// land in one stretch of consecutive addresses.  The other entries keep
// A^T's order (bpos = pinv; their lidx is not read).  One workgroup per
// tile (bucket_kernel) or plan item (bucket_items_kernel).
// One run of cnt <= kCap entries of A^T at base: sorts the pairs (perm[base
// + e], e) by A's entry index in key[] (a bitonic network over the next
// power of two, padded with the largest key), then entry k of rank r gets
// bpos[k] = base + r and lidx[base + r] = its offset e.  Every thread of the
// workgroup takes part.
__device__ void bucket_run(int64_t *key, const int32_t *__restrict__ perm, int64_t base, int cnt,
                           int64_t nnz, int32_t *__restrict__ bpos, uint16_t *__restrict__ lidx) {
    const int tid = threadIdx.x;
    int m = 1;
    while (m < cnt) m <<= 1;
    for (int e = tid; e < m; e += kSetupThreads)
        key[e] = e < cnt ? ((int64_t)perm[base + e] << 16) | e : INT64_MAX;
    __syncthreads();
    for (int size = 2; size <= m; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < m / 2; i += kSetupThreads) {
                const int a = 2 * i - (i & (stride - 1)), b = a + stride;
                const int64_t ka = key[a], kb = key[b];
                if ((ka > kb) == ((a & size) == 0)) {
                    key[a] = kb;
                    key[b] = ka;
                }
            }
            __syncthreads();
        }
    }
    for (int r = tid; r < cnt; r += kSetupThreads) {
        const int64_t kv = key[r];
        if ((kv >> 16) < nnz) bpos[kv >> 16] = (int32_t)(base + r);
        lidx[base + r] = (uint16_t)(kv & 0xFFFF);
    }
}

template <typename IT>
__global__ __launch_bounds__(kSetupThreads) void bucket_kernel(const IT *__restrict__ rp_t,
                                                               const int32_t *__restrict__ perm,
                                                               const uint8_t *__restrict__ planned,
                                                               int64_t n, int64_t nnz,
                                                               int32_t *__restrict__ bpos,
                                                               uint16_t *__restrict__ lidx) {
    static_assert(kCap <= 65536, "offsets inside a tile fit 16 bits");
    __shared__ int64_t key[kCap];
    const int tid = threadIdx.x;
    const int64_t tt = blockIdx.x;
    const int64_t row0 = tt * kTileRows;
    const int64_t rows = n - row0 < kTileRows ? n - row0 : kTileRows;
    const int64_t base = (int64_t)rp_t[row0];
    const int64_t cnt = (int64_t)rp_t[row0 + rows] - base;
    if (planned && planned[tt]) return;  // bucket_items_kernel
    if (cnt > kCap) {
        for (int64_t e = tid; e < cnt; e += kSetupThreads) bpos[perm[base + e]] = (int32_t)(base + e);
        return;
    }
    bucket_run(key, perm, base, (int)cnt, nnz, bpos, lidx);
}

// The same for the tiles A^T's row plan covers, item by item: a short block
// (whole rows, at most kPlanCap entries) is listed in A's entry order; a
// long row's chunk is in A's order already (a row of A^T lists its entries
// by ascending row of A), so there bpos = pinv.
__global__ __launch_bounds__(kSetupThreads) void bucket_items_kernel(
    const PlanItem *__restrict__ items, const int32_t *__restrict__ perm, int64_t nnz,
    int32_t *__restrict__ bpos, uint16_t *__restrict__ lidx) {
    static_assert(kPlanCap <= kCap, "a short block fits the sort");
    __shared__ int64_t key[kCap];
    const PlanItem it = items[blockIdx.x];
    const int64_t cnt = it.e1 - it.e0;
    if (it.kind != 0) {
        for (int64_t e = threadIdx.x; e < cnt; e += kSetupThreads)
            bpos[perm[it.e0 + e]] = (int32_t)(it.e0 + e);
        return;
    }
    bucket_run(key, perm, it.e0, (int)cnt, nnz, bpos, lidx);
}

template <typename IT>
hipError_t setup_buckets(const IT *rp_t, const int32_t *perm, const RowPlan &plan_t, int64_t n,
                         int64_t nnz, int32_t *bpos, uint16_t *lidx, hipStream_t s) {
    const int64_t nt = (n + kTileRows - 1) / kTileRows;
    const bool ps = plan_t.nitems > 0;
    bucket_kernel<IT><<<(unsigned)nt, kSetupThreads, 0, s>>>(rp_t, perm, ps ? plan_t.tiles : nullptr,
                                                             n, nnz, bpos, lidx);
    if (ps)
        bucket_items_kernel<<<(unsigned)plan_t.nitems, kSetupThreads, 0, s>>>(plan_t.items, perm,
                                                                              nnz, bpos, lidx);
    return hipGetLastError();
}

// Launchers of the single checks, for callers that keep their own flags
// (each raises *flag or atomically maxes *out, which must start at 0); they
// allocate nothing and do not synchronize.
template <typename IT>
hipError_t launch_check_rowptr(const IT *rp, int64_t n, int64_t nnz, int32_t *flag,
                               hipStream_t s) {
    check_rowptr_kernel<IT><<<blocks_for(n), kSetupThreads, 0, s>>>(rp, n, nnz, flag);
    return hipGetLastError();
}

template <typename IT>
hipError_t launch_check_cols_rows(const IT *rp, const int32_t *col, int64_t n, IT *diagpos,
                                  int32_t *flag, hipStream_t s) {
    check_cols_kernel<IT><<<blocks_for(n), kSetupThreads, 0, s>>>(rp, col, n, diagpos, flag);
    return hipGetLastError();
}

template <typename IT>
hipError_t launch_max_row(const IT *rp, int64_t n, int32_t *out, hipStream_t s) {
    const unsigned nb = blocks_for(n) < 512 ? blocks_for(n) : 512;
    max_row_kernel<IT><<<nb, kSetupThreads, 0, s>>>(rp, n, out);
    return hipGetLastError();
}

#define SLA_SETUP_INST(IT)                                                                     \
    template hipError_t launch_check_rowptr<IT>(const IT *, int64_t, int64_t, int32_t *,       \
                                                hipStream_t);                                  \
    template hipError_t launch_check_cols_rows<IT>(const IT *, const int32_t *, int64_t, IT *, \
                                                   int32_t *, hipStream_t);                    \
    template hipError_t launch_max_row<IT>(const IT *, int64_t, int32_t *, hipStream_t);      \
    template hipError_t setup_check_rowptr<IT>(const IT *, int64_t, int64_t, int32_t *,        \
                                               int32_t *, hipStream_t);                        \
    template hipError_t setup_row_index<IT>(const IT *, int64_t, int64_t, int32_t *,           \
                                            int32_t *, hipStream_t);                           \
    template hipError_t setup_check_cols<IT>(const IT *, const int32_t *, int64_t, int64_t,    \
                                             const int32_t *, IT *, int32_t *, int32_t *,      \
                                             hipStream_t);                                     \
    template hipError_t setup_max_row<IT>(const IT *, int64_t, int32_t *, int32_t *,           \
                                          hipStream_t);                                        \
    template hipError_t setup_diag<IT>(const IT *, const int32_t *, int64_t, int32_t *,        \
                                       int32_t *, int32_t *, int32_t *, hipStream_t);          \
    template hipError_t setup_diag_masks<IT>(const IT *, const int32_t *, int64_t,             \
                                             const int32_t *, int32_t, uint16_t *,             \
                                             hipStream_t);                                     \
    template hipError_t setup_col16<IT>(const IT *, const int32_t *, int64_t, int64_t,         \
                                        const int32_t *, int16_t *, int32_t *, int32_t *,      \
                                        hipStream_t);                                          \
    template hipError_t setup_transpose<IT>(const IT *, const int32_t *, int64_t, int64_t,     \
                                            IT *, int32_t *, int32_t *, int32_t *,             \
                                            SetupScratch &, hipStream_t);                         \
    template hipError_t setup_buckets<IT>(const IT *, const int32_t *, const RowPlan &, int64_t, \
                                          int64_t, int32_t *, uint16_t *, hipStream_t);
SLA_SETUP_INST(int32_t)
SLA_SETUP_INST(int64_t)
#undef SLA_SETUP_INST

}  // namespace sla
