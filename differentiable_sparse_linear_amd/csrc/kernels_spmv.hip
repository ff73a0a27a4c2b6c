// Sparse matrix-vector products and the single-pass kernels around them.
//
// SpMV (torch-sla explainer, Methodology section 1: .matvec of the unified
// API; the shared-pattern SparseTensor holds a batch of value arrays):
//   y[s][i] = sum over stored k of row i: values[s][k] * x[s][col[k]].
// Rows are processed in tiles (spmv_tile.h): a tile's entries are read as one
// coalesced run with several independent loads in flight per thread, the
// products are staged in LDS and each row is summed in entry order.
// Gradient on the pattern (Methodology section 2, linear systems):
//   grad[s][k] = -lambda[s][row(k)] * x[s][col(k)].
#include "spmv_tile.h"

namespace sla {

template <typename T, typename IT, int SLOTS, int CM>
__global__ __launch_bounds__(kBlock) void spmv_kernel(const IT *__restrict__ rp, ColArgs ca,
                                                      const T *__restrict__ val, int64_t val_stride,
                                                      const T *__restrict__ x, T *__restrict__ y,
                                                      int64_t n, int64_t vec_stride) {
    __shared__ RowLds<T, IT> sm;
    const int sys = blockIdx.y;
    const gptr<const T> v = glb(val + (int64_t)sys * val_stride);
    const gptr<const T> xs = glb(x + (int64_t)sys * vec_stride);
    const gptr<T> ys = glb(y + (int64_t)sys * vec_stride);
    spmv_rows<T, IT, SLOTS, SLOTS>(
        xcd_tiles(tiles_of(n)), n, glb(rp), col_src<CM>(ca), sm, [&](IT k) { return v[k]; },
        [&](int32_t c) { return xs[c]; }, PlainGather(), NoOwn(),
        [&](int64_t i, T s, int, T) { ys[i] = s; }, NoPre(), NoPost());
}

// y = A^T x through the transpose map: rp/col describe A^T and the value of
// A^T entry kt is val[perm[kt]].
template <typename T, typename IT, int SLOTS, int CM>
__global__ __launch_bounds__(kBlock) void spmv_perm_kernel(
    const IT *__restrict__ rp, ColArgs ca, const int32_t *__restrict__ perm,
    const T *__restrict__ val, int64_t val_stride, const T *__restrict__ x, T *__restrict__ y,
    int64_t n, int64_t vec_stride) {
    __shared__ RowLds<T, IT> sm;
    const int sys = blockIdx.y;
    const gptr<const T> v = glb(val + (int64_t)sys * val_stride);
    const gptr<const T> xs = glb(x + (int64_t)sys * vec_stride);
    const gptr<T> ys = glb(y + (int64_t)sys * vec_stride);
    const gptr<const int32_t> pm = glb(perm);
    spmv_rows<T, IT, SLOTS, SLOTS>(
        xcd_tiles(tiles_of(n)), n, glb(rp), col_src<CM>(ca), sm, [&](IT k) { return v[pm[k]]; },
        [&](int32_t c) { return xs[c]; }, PlainGather(), NoOwn(),
        [&](int64_t i, T s, int, T) { ys[i] = s; }, NoPre(), NoPost());
}

// y = A^T x for a pattern with per-row diagonal masks, read from A's own
// rows (no transpose map): row i of A^T holds A[j][i] for j = i - dlt[q],
// stored when bit q of msk[j] is set, at position rp[j] + (set bits of
// msk[j] below q).  q runs downwards, so the terms are added in ascending j,
// the column order of A^T's row.  NDT >= the pattern's diagonal count; all
// NDT slots are unrolled so every mask and row-pointer load of a row is in
// flight before its values are gathered.
template <typename T, typename IT, int NDT>
__global__ __launch_bounds__(kBlock) void spmv_t_diag_kernel(const IT *__restrict__ rp, ColArgs ca,
                                                             const T *__restrict__ val,
                                                             int64_t val_stride,
                                                             const T *__restrict__ x,
                                                             T *__restrict__ y, int64_t n,
                                                             int64_t vec_stride) {
    const int sys = blockIdx.y;
    const gptr<const T> v = glb(val + (int64_t)sys * val_stride);
    const gptr<const T> xs = glb(x + (int64_t)sys * vec_stride);
    const gptr<T> ys = glb(y + (int64_t)sys * vec_stride);
    const gptr<const uint16_t> msk = glb(ca.msk);
    const gptr<const IT> rpg = glb(rp);
    const int nd = ca.nd;
    int32_t dl[NDT];
#pragma unroll
    for (int q = 0; q < NDT; ++q) dl[q] = q < nd ? ca.dlt[q] : 0;
    const TileRange tr = xcd_tiles(tiles_of(n));
    for (int64_t t = tr.first; t < tr.end; t += tr.stride) {
        const int64_t i = t * kTileRows + threadIdx.x;
        if (i >= n) continue;
        bool on[NDT];
        int64_t jj[NDT];
        IT k[NDT];
#pragma unroll
        for (int q = 0; q < NDT; ++q) {
            const int64_t j = i - dl[q];
            on[q] = q < nd && j >= 0 && j < n;
            jj[q] = on[q] ? j : i;
        }
#pragma unroll
        for (int q = 0; q < NDT; ++q) {
            const uint32_t m = msk[jj[q]];
            on[q] = on[q] && ((m >> q) & 1u);
            k[q] = rpg[jj[q]] + (IT)__builtin_popcount(m & ((1u << q) - 1u));
        }
        T s = T(0);
#pragma unroll
        for (int q = NDT - 1; q >= 0; --q) {
            if (on[q]) s = fma(v[k[q]], xs[jj[q]], s);
        }
        ys[i] = s;
    }
}

// grad[k] = -lambda[row(k)] * x[col[k]] (NEG; the solve's gradient on the
// pattern) or g[row(k)] * x[col[k]] (the product's).  Short tiles: each thread marks the
// tile-local row of its row's entries in LDS (with diagonal masks also their
// columns, from the mask's set bits), then the entries are written as one
// coalesced run.  Tiles with long rows: one wavefront per row.
template <typename T, typename IT, bool NEG, int CM>
__global__ __launch_bounds__(kBlock) void grad_kernel(const IT *__restrict__ rp, ColArgs ca,
                                                      const T *__restrict__ lam,
                                                      const T *__restrict__ x, T *__restrict__ grad,
                                                      int64_t n, int64_t nnz) {
    constexpr bool kDiag = CM == kColDiag;
    __shared__ IT srp[kTileRows + 1];
    __shared__ T slam[kTileRows];
    __shared__ uint16_t rid[kCap];
    __shared__ int32_t scol[kDiag ? kCap : 1];
    __shared__ int32_t dtab[kMaxDiags];
    const int sys = blockIdx.y;
    const ColSrc<CM> col = col_src<CM>(ca);
    if (kDiag && threadIdx.x < kMaxDiags) dtab[threadIdx.x] = ca.dlt[threadIdx.x];
    lam += (int64_t)sys * n;
    x += (int64_t)sys * n;
    grad += (int64_t)sys * nnz;
    const int tid = threadIdx.x;
    const TileRange tr = xcd_tiles(tiles_of(n));
    for (int64_t t = tr.first; t < tr.end; t += tr.stride) {
        const int64_t row0 = t * kTileRows;
        const int64_t left = n - row0;
        const int rows = left < kTileRows ? (int)left : kTileRows;
        if (tid < rows) {
            srp[tid] = rp[row0 + tid];
            slam[tid] = lam[row0 + tid];
        }
        if (tid == 0) srp[rows] = rp[row0 + rows];
        __syncthreads();
        const IT base = srp[0];
        const int64_t cnt = (int64_t)(srp[rows] - base);
        if (cnt <= kCap) {
            if (tid < rows) {
                uint32_t m = kDiag ? (uint32_t)col.msk[row0 + tid] : 0u;
                for (int e = (int)(srp[tid] - base); e < (int)(srp[tid + 1] - base); ++e) {
                    rid[e] = (uint16_t)tid;
                    if (kDiag) {
                        scol[e] = (int32_t)(row0 + tid) + dtab[__builtin_ctz(m | 0x8000u)];
                        m &= m - 1u;
                    }
                }
            }
            __syncthreads();
            int32_t c[kEpt];
#pragma unroll
            for (int j = 0; j < kEpt; ++j) {
                const int e = tid + j * kBlock;
                if (e < cnt) c[j] = kDiag ? scol[e] : col(base + e, row0);
            }
#pragma unroll
            for (int j = 0; j < kEpt; ++j) {
                const int e = tid + j * kBlock;
                if (e < cnt) {
                    const T g = slam[rid[e]] * x[c[j]];
                    grad[base + e] = NEG ? -g : g;
                }
            }
        } else {
            const int lane = tid & 63, wave = tid >> 6;
            for (int r = wave; r < rows; r += kWaves) {
                const T li = slam[r];
                const IT lo = srp[r], hi = srp[r + 1];
                const uint32_t mr = kDiag ? (uint32_t)col.msk[row0 + r] : 0u;
                for (IT k = lo + lane; k < hi; k += 64) {
                    const int32_t c = kDiag ? (int32_t)(row0 + r) + dtab[nth_bit(mr, (int)(k - lo))]
                                            : col(k, row0);
                    const T g = li * x[c];
                    grad[k] = NEG ? -g : g;
                }
            }
        }
        __syncthreads();
    }
}

template <typename T>
__global__ __launch_bounds__(kBlock) void gather_kernel(const int32_t *__restrict__ perm,
                                                        const T *__restrict__ val,
                                                        T *__restrict__ out, int64_t nnz) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x; k < nnz; k += stride)
        out[k] = val[perm[k]];
}

// out[q * n + i] = row i's entry on diagonal q, 0 where bit q of msk[i] is
// clear.  The row's entries are stored in ascending column order, which is
// ascending q, so the k-th set bit takes the k-th entry.  System blockIdx.y
// reads val + y * val_stride and writes out + y * nd * n.
template <typename T, typename IT>
__global__ __launch_bounds__(kBlock) void dia_pack_kernel(const IT *__restrict__ rp,
                                                          const uint16_t *__restrict__ msk, int nd,
                                                          const T *__restrict__ val,
                                                          int64_t val_stride,
                                                          T *__restrict__ out, int64_t n) {
    val += (int64_t)blockIdx.y * val_stride;
    out += (int64_t)blockIdx.y * nd * n;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride) {
        uint32_t m = msk[i];
        IT k = rp[i];
        for (int q = 0; q < nd; ++q, m >>= 1) {
            T v = T(0);
            if (m & 1u) v = val[k++];
            out[(int64_t)q * n + i] = v;
        }
    }
}

// System blockIdx.y: values val + y * val_stride, dinv + y * n, state st + y.
template <typename T, typename IT>
__global__ __launch_bounds__(kBlock) void dinv_kernel(const IT *__restrict__ diagpos,
                                                      const T *__restrict__ val,
                                                      int64_t val_stride, T *__restrict__ dinv,
                                                      int64_t n, SolveState *st) {
    val += (int64_t)blockIdx.y * val_stride;
    dinv += (int64_t)blockIdx.y * n;
    st += blockIdx.y;
    const TileRange tr = xcd_tiles(tiles_of(n));
    int bad = 0;
    for (int64_t t = tr.first; t < tr.end; t += tr.stride) {
        const int64_t i = t * kTileRows + threadIdx.x;
        if (i < n) {
            const T d = val[diagpos[i]];
            bad |= (d == T(0));
            dinv[i] = T(1) / d;
        }
    }
    if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(&st->zero_diag, 1);
}

// x + y * n = 0 for system y = blockIdx.y when its state asks for it.
template <typename T>
__global__ __launch_bounds__(kBlock) void zero_if_kernel(const SolveState *st, T *x, int64_t n) {
    st += blockIdx.y;
    x += (int64_t)blockIdx.y * n;
    if (!st->zero_x) return;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride) x[i] = T(0);
}

// ------------------------------------------------------------------ launchers

template <typename T, typename IT>
hipError_t launch_spmv(int slots, const IT *rp, const ColArgs &ca, const T *val,
                       int64_t val_stride, const T *x, T *y, int64_t n, int64_t vec_stride,
                       int batch, hipStream_t s) {
    const dim3 grid(grid_for_tiles(tiles_of(n)), batch);
    SLA_DISPATCH_CM(ca.mode, SLA_DISPATCH_SLOTS(slots, spmv_kernel<T, IT, kS, kC>
                                                <<<grid, kBlock, 0, s>>>(rp, ca, val, val_stride,
                                                                         x, y, n, vec_stride)));
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_spmv_perm(int slots, const IT *rp, const ColArgs &ca, const int32_t *perm,
                            const T *val, int64_t val_stride, const T *x, T *y, int64_t n,
                            int64_t vec_stride, int batch, hipStream_t s) {
    const dim3 grid(grid_for_tiles(tiles_of(n)), batch);
    SLA_DISPATCH_CM(ca.mode, SLA_DISPATCH_SLOTS(slots, spmv_perm_kernel<T, IT, kS, kC>
                                                <<<grid, kBlock, 0, s>>>(rp, ca, perm, val,
                                                                         val_stride, x, y, n,
                                                                         vec_stride)));
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_spmv_t_diag(const IT *rp, const ColArgs &ca, const T *val, int64_t val_stride,
                              const T *x, T *y, int64_t n, int64_t vec_stride, int batch,
                              hipStream_t s) {
    const dim3 grid(grid_for_tiles(tiles_of(n)), batch);
    if (ca.nd <= 4)
        spmv_t_diag_kernel<T, IT, 4><<<grid, kBlock, 0, s>>>(rp, ca, val, val_stride, x, y, n,
                                                             vec_stride);
    else if (ca.nd <= 8)
        spmv_t_diag_kernel<T, IT, 8><<<grid, kBlock, 0, s>>>(rp, ca, val, val_stride, x, y, n,
                                                             vec_stride);
    else
        spmv_t_diag_kernel<T, IT, kMaxDiags><<<grid, kBlock, 0, s>>>(rp, ca, val, val_stride, x,
                                                                     y, n, vec_stride);
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_grad(const IT *rp, const ColArgs &ca, const T *lam, const T *x, T *grad,
                       int64_t n, int64_t nnz, int batch, bool neg, hipStream_t s) {
    const dim3 grid(grid_for_tiles(tiles_of(n)), batch);
    SLA_DISPATCH_CM(ca.mode, if (neg) {
        grad_kernel<T, IT, true, kC><<<grid, kBlock, 0, s>>>(rp, ca, lam, x, grad, n, nnz);
    } else {
        grad_kernel<T, IT, false, kC><<<grid, kBlock, 0, s>>>(rp, ca, lam, x, grad, n, nnz);
    });
    return hipGetLastError();
}

template <typename T>
hipError_t launch_gather(const int32_t *perm, const T *val, T *out, int64_t nnz, hipStream_t s) {
    int64_t blocks = (nnz + kBlock - 1) / kBlock;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    gather_kernel<T><<<(unsigned)blocks, kBlock, 0, s>>>(perm, val, out, nnz);
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_dia_pack(const IT *rp, const uint16_t *msk, int nd, const T *val,
                           int64_t val_stride, T *out, int64_t n, int nsys, hipStream_t s) {
    int64_t blocks = (n + kBlock - 1) / kBlock;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    dia_pack_kernel<T, IT><<<dim3((unsigned)blocks, nsys), kBlock, 0, s>>>(rp, msk, nd, val,
                                                                           val_stride, out, n);
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_dinv(const IT *diagpos, const T *val, int64_t val_stride, T *dinv, int64_t n,
                       SolveState *st, int nsys, hipStream_t s) {
    dinv_kernel<T, IT><<<dim3(grid_for_tiles(tiles_of(n)), nsys), kBlock, 0, s>>>(
        diagpos, val, val_stride, dinv, n, st);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_zero_if(const SolveState *st, T *x, int64_t n, int nsys, hipStream_t s) {
    int64_t blocks = (n + kBlock - 1) / kBlock;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    zero_if_kernel<T><<<dim3((unsigned)blocks, nsys), kBlock, 0, s>>>(st, x, n);
    return hipGetLastError();
}

#define SLA_INST(T, IT)                                                                         \
    template hipError_t launch_spmv<T, IT>(int, const IT *, const ColArgs &, const T *, int64_t, \
                                           const T *, T *, int64_t, int64_t, int, hipStream_t);  \
    template hipError_t launch_spmv_perm<T, IT>(int, const IT *, const ColArgs &,               \
                                                const int32_t *, const T *, int64_t, const T *,  \
                                                T *, int64_t, int64_t, int, hipStream_t);        \
    template hipError_t launch_spmv_t_diag<T, IT>(const IT *, const ColArgs &, const T *,       \
                                                  int64_t, const T *, T *, int64_t, int64_t,     \
                                                  int, hipStream_t);                             \
    template hipError_t launch_grad<T, IT>(const IT *, const ColArgs &, const T *, const T *,   \
                                           T *, int64_t, int64_t, int, bool, hipStream_t);      \
    template hipError_t launch_dinv<T, IT>(const IT *, const T *, int64_t, T *, int64_t,        \
                                           SolveState *, int, hipStream_t);                      \
    template hipError_t launch_dia_pack<T, IT>(const IT *, const uint16_t *, int, const T *,    \
                                               int64_t, T *, int64_t, int, hipStream_t);

SLA_INST(float, int32_t)
SLA_INST(float, int64_t)
SLA_INST(double, int32_t)
SLA_INST(double, int64_t)
template hipError_t launch_gather<float>(const int32_t *, const float *, float *, int64_t,
                                         hipStream_t);
template hipError_t launch_gather<double>(const int32_t *, const double *, double *, int64_t,
                                          hipStream_t);
template hipError_t launch_zero_if<float>(const SolveState *, float *, int64_t, int, hipStream_t);
template hipError_t launch_zero_if<double>(const SolveState *, double *, int64_t, int,
                                           hipStream_t);

}  // namespace sla
