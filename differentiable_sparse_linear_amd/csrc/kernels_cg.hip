// Conjugate gradients with an optional Jacobi preconditioner M = diag(A)
// (torch-sla explainer, Methodology section 1 and the Significance section:
// the native backend is an iterative solver with a Jacobi preconditioner;
// steps as in Saad, Iterative Methods for Sparse Linear Systems, Alg. 9.1).
//
// Grid path, two kernels per iteration over one system:
//   cg_spmv:   stop test on r_k; beta = rho_k / rho_{k-1};
//              p_k = z_k + beta p_{k-1} (p_0 = z_0) evaluated while gathering,
//              q = A p_k, stored p_k and q; partial p.q
//   cg_update: alpha = rho_k / p.q (p.q <= 0: breakdown); x += alpha p,
//              r -= alpha q, z = M^-1 r; partials r.z and r.r
// Each kernel stores per-block partial sums with plain stores; every block
// of the next kernel adds them in block order, so all blocks derive the same
// scalars and no grid-wide fence is needed (a release at agent scope costs an
// L2 write-back per block on a multi-XCD part).  p is double-buffered by
// iteration parity because cg_spmv reads the old p at neighbouring rows while
// it writes the new one.  Every kernel returns at entry once the device-side
// `done` flag is set, so the host can enqueue many iterations (HIP graph
// replays) and poll rarely.
//
// Block path: one 1024-thread workgroup runs the whole solve of one small
// system (n <= 4096): vectors live in registers, the search direction in LDS
// for the gathers, reductions in LDS; no grid-wide synchronisation and no
// per-iteration launches (the pages note that launch overhead hurts iterative
// solvers on small problems: Problem statement, backend fragmentation).
#include "spmv_tile.h"

namespace sla {

template <typename T>
__device__ __forceinline__ T fmaT(T a, T b, T c) {
    return fma(a, b, c);
}

// r = b - A x0 (or b with x = 0), z = M^-1 r; partials r.z, r.r, b.b.
template <typename T, typename IT, bool JAC>
__global__ __launch_bounds__(kBlock) void cg_init_kernel(const IterArgs<T, IT> *__restrict__ A) {
    const int64_t n = A->n;
    const T *b = A->b;
    T *x = A->x;
    T *r = A->r;
    T *z = A->z;
    const T *dinv = A->dinv;
    const T *ax0 = A->q;  // A x0 when use_x0
    const bool x0 = A->use_x0 != 0;
    double rz = 0.0, rr = 0.0, bb = 0.0;
    const TileRange tr = xcd_tiles(tiles_of(n));
    for (int64_t t = tr.first; t < tr.end; t += tr.stride) {
        const int64_t i = t * kTileRows + threadIdx.x;
        if (i < n) {
            const T bi = b[i];
            T ri = bi;
            if (x0)
                ri = bi - ax0[i];
            else
                x[i] = T(0);
            r[i] = ri;
            T zi = ri;
            if (JAC) {
                zi = dinv[i] * ri;
                z[i] = zi;
            }
            rz += (double)ri * (double)zi;
            rr += (double)ri * (double)ri;
            bb += (double)bi * (double)bi;
        }
    }
    double v[3] = {rz, rr, bb};
    const int slot[3] = {kCgRZ, kCgRR, kCgBB};
    store_partials<3>(v, A->part, slot);
}

// Iteration k (k = iter_a): stop test on r_k, beta_k = rho_k / rho_{k-1},
// p_k = z_k + beta_k p_{k-1} evaluated while gathering, q = A p_k,
// partial p_k.q.
template <typename T, typename IT, bool JAC>
__global__ __launch_bounds__(kBlock) void cg_spmv_kernel(const IterArgs<T, IT> *__restrict__ A) {
    SolveState *st = A->st;
    if (load_done(st)) return;
    const int it = st->iter_a;
    double tot[3];
    {
        const int slot[3] = {kCgRZ, kCgRR, kCgBB};
        load_totals<3>(A->part, gridDim.x, slot, tot);
    }
    const double rho = tot[0], rr = tot[1];
    const double bb = it == 0 ? tot[2] : st->bb;
    // stop tests on the residual left by the previous update (or the start)
    if (it == 0 && st->zero_diag) {
        finish(st, SLA_ERR_ZERO_DIAG, 0, rr);
        return;
    }
    if (it == 0 && bb == 0.0) {
        if (block0()) st->zero_x = A->use_x0 ? 1 : 0;
        finish(st, SLA_OK, 0, 0.0);
        return;
    }
    if (sqrt(rr) <= A->tol * sqrt(bb)) {
        finish(st, SLA_OK, it, rr);
        return;
    }
    if (it >= A->maxit) {
        finish(st, SLA_NOT_CONVERGED, it, rr);
        return;
    }
    const bool first = (it == 0);
    const T beta = first ? T(0) : (T)(rho / st->rho[(it + 1) & 1]);
    if (block0()) {
        st->rho[it & 1] = rho;
        st->iter_b = it;
        st->spmv += (first && A->use_x0) ? 2 : 1;  // counts the A x0 product
        st->nfused += 1;
        if (first) st->bb = bb;
    }
    const T *__restrict__ zz = JAC ? A->z : A->r;
    const T *__restrict__ pold = A->p[it & 1];
    T *__restrict__ pnew = A->p[(it + 1) & 1];
    const IT *__restrict__ rp = A->rp;
    const int32_t *__restrict__ col = A->col;
    const T *__restrict__ val = A->val;
    T *__restrict__ q = A->q;
    const int64_t n = A->n;
    __shared__ TileLds<T, IT> sm;
    double pq = 0.0;
    auto pdir = [&](int64_t c) { return first ? zz[c] : fmaT(beta, pold[c], zz[c]); };
    const TileRange tr = xcd_tiles(tiles_of(n));
    for (int64_t t = tr.first; t < tr.end; t += tr.stride)
        spmv_tile<T, IT>(
            t, n, rp, col, sm, [&](IT k) { return val[k]; }, [&](int32_t c) { return pdir(c); },
            [&](int64_t i, T acc) {
                const T pi = pdir(i);
                pnew[i] = pi;
                q[i] = acc;
                pq += (double)pi * (double)acc;
            });
    double v[1] = {pq};
    const int slot[1] = {kCgPQ};
    store_partials<1>(v, A->part, slot);
}

// Iteration k (k = iter_b): alpha = rho_k / p.q (p.q <= 0: breakdown);
// x += alpha p, r -= alpha q, z = M^-1 r; partials r.z and r.r.
template <typename T, typename IT, bool JAC>
__global__ __launch_bounds__(kBlock) void cg_update_kernel(const IterArgs<T, IT> *__restrict__ A) {
    SolveState *st = A->st;
    if (load_done(st)) return;
    const int it = st->iter_b;
    double tot[1];
    {
        const int slot[1] = {kCgPQ};
        load_totals<1>(A->part, gridDim.x, slot, tot);
    }
    if (!(tot[0] > 0.0)) {
        finish(st, SLA_BREAKDOWN, it, 0.0);
        return;
    }
    const T alpha = (T)(st->rho[it & 1] / tot[0]);
    if (block0()) st->iter_a = it + 1;
    const T *__restrict__ p = A->p[(it + 1) & 1];
    const T *__restrict__ q = A->q;
    const T *__restrict__ dinv = A->dinv;
    T *__restrict__ x = A->x;
    T *__restrict__ r = A->r;
    T *__restrict__ z = A->z;
    const int64_t n = A->n;
    double rz = 0.0, rr = 0.0;
    const TileRange tr = xcd_tiles(tiles_of(n));
    for (int64_t t = tr.first; t < tr.end; t += tr.stride) {
        const int64_t i = t * kTileRows + threadIdx.x;
        if (i < n) {
            x[i] = fmaT(alpha, p[i], x[i]);
            const T ri = fmaT(-alpha, q[i], r[i]);
            r[i] = ri;
            T zi = ri;
            if (JAC) {
                zi = dinv[i] * ri;
                z[i] = zi;
            }
            rz += (double)ri * (double)zi;
            rr += (double)ri * (double)ri;
        }
    }
    double v[2] = {rz, rr};
    const int slot[2] = {kCgRZ, kCgRR};
    store_partials<2>(v, A->part, slot);
}

// ------------------------------------------------------------ block path

constexpr int kBW = kBlockSolveThreads / 64;  // waves per workgroup
constexpr int kMaxRpt = kBlockSolveMaxN / kBlockSolveThreads;

// Sum over the workgroup; every thread receives the same, order-fixed total.
template <int NR>
__device__ __forceinline__ void block_sum(double (&v)[NR], double (*slots)[kBW]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const double w = wave_sum(v[r]);
        if (lane == 0) slots[r][wave] = w;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        double s = 0.0;
#pragma unroll
        for (int w = 0; w < kBW; ++w) s += slots[r][w];
        v[r] = s;
    }
}

// Row ownership: the SpMV sweeps rows in passes of RPP = 1024/G rows, one row
// per G-lane group; pass `ps` covers rows ps*RPP + group.  The lane
// (ps % G) of that group keeps the row's vector entries in register slot
// ps / G, so the product lands in registers without an LDS round trip.
template <typename T, typename IT, int G>
__global__ __launch_bounds__(kBlockSolveThreads) void block_cg_kernel(BlockCgParams P) {
    extern __shared__ unsigned char lds_raw[];
    T *ps = reinterpret_cast<T *>(lds_raw);  // search direction (or x0), [n]
    __shared__ double slots[4][3][kBW];
    constexpr int RPP = kBlockSolveThreads / G;
    const int sys = blockIdx.x;
    const int64_t n = P.n, nnz = P.nnz;
    const T *__restrict__ val = reinterpret_cast<const T *>(P.val) + (int64_t)sys * nnz;
    const T *__restrict__ b = reinterpret_cast<const T *>(P.b) + (int64_t)sys * n;
    T *__restrict__ x = reinterpret_cast<T *>(P.x) + (int64_t)sys * n;
    const IT *__restrict__ rp = reinterpret_cast<const IT *>(P.rp);
    const IT *__restrict__ dpos = reinterpret_cast<const IT *>(P.diagpos);
    const int32_t *__restrict__ col = P.col;
    SolveState *st = P.st + sys;
    const int lane = threadIdx.x & (G - 1);
    const int grp = threadIdx.x / G;
    const int npass = (int)((n + RPP - 1) / RPP);

    T xr[kMaxRpt], rr[kMaxRpt], pr[kMaxRpt], qr[kMaxRpt], dr[kMaxRpt];
    int bad = 0;
#pragma unroll
    for (int j = 0; j < kMaxRpt; ++j) {
        const int64_t i = (int64_t)(j * G + lane) * RPP + grp;
        xr[j] = rr[j] = pr[j] = qr[j] = T(0);
        dr[j] = T(1);
        if (j * G + lane < npass && i < n) {
            if (P.use_x0) xr[j] = x[i];
            if (P.jac) {
                const T d = val[dpos[i]];
                bad |= (d == T(0));
                dr[j] = T(1) / d;
            }
        }
    }

    // q = A v for v staged in ps; results go to the owning lane's register.
    auto spmv = [&](T(&out)[kMaxRpt]) {
#pragma unroll
        for (int j = 0; j < kMaxRpt; ++j) {
#pragma unroll
            for (int l = 0; l < G; ++l) {
                const int pss = j * G + l;
                if (pss < npass) {
                    const int64_t i = (int64_t)pss * RPP + grp;
                    T acc = T(0);
                    if (i < n) {
                        const IT e = rp[i + 1];
                        for (IT k = rp[i] + lane; k < e; k += G) acc += val[k] * ps[col[k]];
                    }
                    acc = group_sum<G>(acc);
                    if (lane == l) out[j] = acc;
                }
            }
        }
    };
    auto stage = [&](const T(&v)[kMaxRpt]) {
#pragma unroll
        for (int j = 0; j < kMaxRpt; ++j) {
            const int64_t i = (int64_t)(j * G + lane) * RPP + grp;
            if (j * G + lane < npass && i < n) ps[i] = v[j];
        }
    };

    if (P.use_x0) {
        stage(xr);
        __syncthreads();
        spmv(qr);
        __syncthreads();
    }
    double r0[3] = {0.0, 0.0, 0.0};  // r.z, r.r, b.b
#pragma unroll
    for (int j = 0; j < kMaxRpt; ++j) {
        const int64_t i = (int64_t)(j * G + lane) * RPP + grp;
        if (j * G + lane < npass && i < n) {
            const T bi = b[i];
            const T ri = P.use_x0 ? bi - qr[j] : bi;
            rr[j] = ri;
            const T zi = P.jac ? dr[j] * ri : ri;
            pr[j] = zi;
            r0[0] += (double)ri * (double)zi;
            r0[1] += (double)ri * (double)ri;
            r0[2] += (double)bi * (double)bi;
        }
    }
    block_sum<3>(r0, slots[0]);
    const int any_bad = __syncthreads_or(bad);
    double rho = r0[0], rnorm2 = r0[1];
    const double bb = r0[2];
    const double thresh = P.tol * sqrt(bb);
    int status = SLA_NOT_CONVERGED, it = 0;
    bool zero_x = false;
    if (any_bad) {
        status = SLA_ERR_ZERO_DIAG;
    } else if (bb == 0.0) {
        status = SLA_OK;
        zero_x = true;
    } else if (sqrt(rnorm2) <= thresh) {
        status = SLA_OK;
    } else {
        int slot = 1;
        while (it < P.maxit) {
            stage(pr);
            __syncthreads();
            spmv(qr);
            double pq[1] = {0.0};
#pragma unroll
            for (int j = 0; j < kMaxRpt; ++j) pq[0] += (double)pr[j] * (double)qr[j];
            block_sum<1>(pq, slots[slot]);
            slot = (slot + 1) & 3;
            if (!(pq[0] > 0.0)) {
                status = SLA_BREAKDOWN;
                break;
            }
            const T alpha = (T)(rho / pq[0]);
            double red[2] = {0.0, 0.0};
            T zr[kMaxRpt];
#pragma unroll
            for (int j = 0; j < kMaxRpt; ++j) {
                xr[j] = fmaT(alpha, pr[j], xr[j]);
                rr[j] = fmaT(-alpha, qr[j], rr[j]);
                zr[j] = P.jac ? dr[j] * rr[j] : rr[j];
                red[0] += (double)rr[j] * (double)zr[j];
                red[1] += (double)rr[j] * (double)rr[j];
            }
            block_sum<2>(red, slots[slot]);
            slot = (slot + 1) & 3;
            ++it;
            rnorm2 = red[1];
            if (sqrt(red[1]) <= thresh) {
                status = SLA_OK;
                break;
            }
            const T beta = (T)(red[0] / rho);
            rho = red[0];
#pragma unroll
            for (int j = 0; j < kMaxRpt; ++j) pr[j] = fmaT(beta, pr[j], zr[j]);
            __syncthreads();  // every gather of the old direction is done
        }
    }
#pragma unroll
    for (int j = 0; j < kMaxRpt; ++j) {
        const int64_t i = (int64_t)(j * G + lane) * RPP + grp;
        if (j * G + lane < npass && i < n) x[i] = zero_x ? T(0) : xr[j];
    }
    if (threadIdx.x == 0) {
        st->iter = it;
        st->spmv = it + (P.use_x0 ? 1 : 0);
        st->status = status;
        st->rr = rnorm2;
        st->bb = bb;
        st->done = 1;
    }
}

// ------------------------------------------------------------------ launchers

#define SLA_DISPATCH_G(G, ...)                      \
    switch (G) {                                    \
        case 2: { constexpr int kG = 2; __VA_ARGS__; } break;   \
        case 4: { constexpr int kG = 4; __VA_ARGS__; } break;   \
        case 8: { constexpr int kG = 8; __VA_ARGS__; } break;   \
        case 16: { constexpr int kG = 16; __VA_ARGS__; } break; \
        case 32: { constexpr int kG = 32; __VA_ARGS__; } break; \
        default: { constexpr int kG = 64; __VA_ARGS__; } break; \
    }

template <typename T, typename IT>
hipError_t launch_cg_init(bool jac, const IterArgs<T, IT> *a, int64_t n, hipStream_t s) {
    const int grid = grid_for_tiles(tiles_of(n));
    if (jac)
        cg_init_kernel<T, IT, true><<<grid, kBlock, 0, s>>>(a);
    else
        cg_init_kernel<T, IT, false><<<grid, kBlock, 0, s>>>(a);
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_cg_spmv(int, bool jac, const IterArgs<T, IT> *a, int64_t n, hipStream_t s) {
    const int grid = grid_for_tiles(tiles_of(n));
    if (jac)
        cg_spmv_kernel<T, IT, true><<<grid, kBlock, 0, s>>>(a);
    else
        cg_spmv_kernel<T, IT, false><<<grid, kBlock, 0, s>>>(a);
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_cg_update(bool jac, const IterArgs<T, IT> *a, int64_t n, hipStream_t s) {
    const int grid = grid_for_tiles(tiles_of(n));
    if (jac)
        cg_update_kernel<T, IT, true><<<grid, kBlock, 0, s>>>(a);
    else
        cg_update_kernel<T, IT, false><<<grid, kBlock, 0, s>>>(a);
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_block_cg(int G, const BlockCgParams &p, int batch, hipStream_t s) {
    const size_t lds = (size_t)p.n * sizeof(T);
    switch (G) {
        case 2:
        case 4:
            block_cg_kernel<T, IT, 4><<<batch, kBlockSolveThreads, lds, s>>>(p);
            break;
        case 8:
            block_cg_kernel<T, IT, 8><<<batch, kBlockSolveThreads, lds, s>>>(p);
            break;
        default:
            block_cg_kernel<T, IT, 16><<<batch, kBlockSolveThreads, lds, s>>>(p);
            break;
    }
    return hipGetLastError();
}

#define SLA_INST(T, IT)                                                                         \
    template hipError_t launch_cg_init<T, IT>(bool, const IterArgs<T, IT> *, int64_t,           \
                                              hipStream_t);                                     \
    template hipError_t launch_cg_spmv<T, IT>(int, bool, const IterArgs<T, IT> *, int64_t,      \
                                              hipStream_t);                                     \
    template hipError_t launch_cg_update<T, IT>(bool, const IterArgs<T, IT> *, int64_t,         \
                                                hipStream_t);                                   \
    template hipError_t launch_block_cg<T, IT>(int, const BlockCgParams &, int, hipStream_t);

SLA_INST(float, int32_t)
SLA_INST(float, int64_t)
SLA_INST(double, int32_t)
SLA_INST(double, int64_t)

}  // namespace sla
