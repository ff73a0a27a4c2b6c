// BiCGStab for nonsymmetric systems (torch-sla explainer, Methodology
// section 1 lists BiCGStab among the iterative solvers; steps of van der
// Vorst, SIAM J. Sci. Stat. Comput. 13, 1992), unpreconditioned, grid path.
//
// Iteration k, three kernels:
//   bicg_pv:     stop tests; rho = rhat.r, beta; p = r + beta (p - omega v)
//                evaluated while gathering, v = A p; partial rhat.v
//   bicg_st:     alpha = rho / rhat.v; s = r - alpha v evaluated while
//                gathering, t = A s; partials t.s, t.t, s.s
//   bicg_update: half step (||s|| <= tol ||b||): x += alpha p; else
//                omega = t.s / t.t, x += alpha p + omega s, r = s - omega t;
//                partials rhat.r and r.r
// Each kernel stores per-block partial sums; every block of the next kernel
// adds them in the same order, so the scalars are identical everywhere and no
// kernel needs a grid-wide fence.  p and v are double-buffered by iteration
// parity (the SpMV kernels read the old vectors at neighbouring rows while
// they write the new ones).
#include "spmv_tile.h"

namespace sla {

template <typename T>
__device__ __forceinline__ T fmaB(T a, T b, T c) {
    return fma(a, b, c);
}

// p_k at one index from r, the previous p and v (p_1 = r)
template <typename T>
__device__ __forceinline__ T pdir(bool first, T beta, T omega, T r, T p, T v) {
    return first ? r : fmaB(beta, fmaB(-omega, v, p), r);
}

// r = rhat = b - A x0 (or b with x = 0); partials r.r (= rhat.r) and b.b.
template <typename T, typename IT>
__global__ __launch_bounds__(kBlock) void bicg_init_kernel(const IterArgs<T, IT> *__restrict__ A) {
    const int64_t n = A->n;
    const T *b = A->b;
    T *x = A->x;
    T *r = A->r;
    T *rh = A->rh;
    const T *ax0 = A->q;
    const bool x0 = A->use_x0 != 0;
    double rr = 0.0, bb = 0.0;
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
            rh[i] = ri;
            rr += (double)ri * (double)ri;
            bb += (double)bi * (double)bi;
        }
    }
    double v[3] = {rr, rr, bb};
    const int slot[3] = {kBiRHR, kBiRR, kBiBB};
    store_partials<3>(v, A->part, slot);
}

// Iteration k (0-based, k = iter_a): a pending half-step exit stops here;
// stop tests on r_k; rho_k = rhat.r_k
// (0: breakdown); beta = (rho_k/rho_{k-1})(alpha_{k-1}/omega_{k-1});
// p = r + beta (p - omega v) evaluated while gathering (p = r at k = 0);
// v = A p; partial rhat.v.
template <typename T, typename IT>
__global__ __launch_bounds__(kBlock) void bicg_pv_kernel(const IterArgs<T, IT> *__restrict__ A) {
    SolveState *st = A->st;
    if (load_done(st)) return;
    const int it = st->iter_a;
    double tot[3];
    {
        const int slot[3] = {kBiRHR, kBiRR, kBiBB};
        load_totals<3>(A->part, gridDim.x, slot, tot);
    }
    if (st->half_exit) {
        finish(st, SLA_OK, it, st->half_ss);
        return;
    }
    const double rho = tot[0], rr = tot[1];
    const double bb = it == 0 ? tot[2] : st->bb;
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
    if (rho == 0.0) {
        finish(st, SLA_BREAKDOWN, it, rr);
        return;
    }
    const bool first = (it == 0);
    const int pv = (it + 1) & 1;  // parity slot of iteration k-1
    const T beta = first ? T(0) : (T)((rho / st->rho[pv]) * (st->alpha[pv] / st->omega[pv]));
    const T omega = first ? T(0) : (T)st->omega[pv];
    if (block0()) {
        st->rho[it & 1] = rho;
        st->iter_b = it;
        st->spmv += (first && A->use_x0) ? 2 : 1;  // counts the A x0 product
        st->nfused += 1;
        if (first) st->bb = bb;
    }
    const T *__restrict__ r = A->r;
    const T *__restrict__ rh = A->rh;
    const T *__restrict__ pold = A->p[it & 1];
    const T *__restrict__ vold = A->v[it & 1];
    T *__restrict__ pnew = A->p[(it + 1) & 1];
    T *__restrict__ vnew = A->v[(it + 1) & 1];
    const IT *__restrict__ rp = A->rp;
    const int32_t *__restrict__ col = A->col;
    const T *__restrict__ val = A->val;
    const int64_t n = A->n;
    __shared__ TileLds<T, IT> sm;
    double rv = 0.0;
    auto pk = [&](int64_t c) { return first ? r[c] : pdir(false, beta, omega, r[c], pold[c], vold[c]); };
    const TileRange tr = xcd_tiles(tiles_of(n));
    for (int64_t t = tr.first; t < tr.end; t += tr.stride)
        spmv_tile<T, IT>(
            t, n, rp, col, sm, [&](IT k) { return val[k]; }, [&](int32_t c) { return pk(c); },
            [&](int64_t i, T acc) {
                pnew[i] = pk(i);
                vnew[i] = acc;
                rv += (double)rh[i] * (double)acc;
            });
    double v[1] = {rv};
    const int slot[1] = {kBiRV};
    store_partials<1>(v, A->part, slot);
}

// Iteration k (k = iter_b): alpha = rho_k / rhat.v (0: breakdown);
// s = r - alpha v evaluated while gathering, t = A s; partials t.s, t.t, s.s.
template <typename T, typename IT>
__global__ __launch_bounds__(kBlock) void bicg_st_kernel(const IterArgs<T, IT> *__restrict__ A) {
    SolveState *st = A->st;
    if (load_done(st)) return;
    const int it = st->iter_b;
    double tot[1];
    {
        const int slot[1] = {kBiRV};
        load_totals<1>(A->part, gridDim.x, slot, tot);
    }
    if (tot[0] == 0.0) {
        finish(st, SLA_BREAKDOWN, it, 0.0);
        return;
    }
    const double alpha_d = st->rho[it & 1] / tot[0];
    const T alpha = (T)alpha_d;
    if (block0()) {
        st->alpha[it & 1] = alpha_d;
        st->iter_c = it;
        st->nfused += 1;
    }
    const T *__restrict__ r = A->r;
    const T *__restrict__ v = A->v[(it + 1) & 1];
    T *__restrict__ s = A->s;
    T *__restrict__ tv = A->t;
    const IT *__restrict__ rp = A->rp;
    const int32_t *__restrict__ col = A->col;
    const T *__restrict__ val = A->val;
    const int64_t n = A->n;
    __shared__ TileLds<T, IT> sm;
    double ts = 0.0, tt = 0.0, ss = 0.0;
    auto sk = [&](int64_t c) { return fmaB(-alpha, v[c], r[c]); };
    const TileRange tr = xcd_tiles(tiles_of(n));
    for (int64_t t = tr.first; t < tr.end; t += tr.stride)
        spmv_tile<T, IT>(
            t, n, rp, col, sm, [&](IT k) { return val[k]; }, [&](int32_t c) { return sk(c); },
            [&](int64_t i, T acc) {
                const T si = sk(i);
                s[i] = si;
                tv[i] = acc;
                ts += (double)acc * (double)si;
                tt += (double)acc * (double)acc;
                ss += (double)si * (double)si;
            });
    double red[3] = {ts, tt, ss};
    const int slot[3] = {kBiTS, kBiTT, kBiSS};
    store_partials<3>(red, A->part, slot);
}

// Iteration k (k = iter_c): half-step exit when ||s|| <= tol ||b||
// (x += alpha p); else omega = t.s / t.t (t.t = 0 or t.s = 0: breakdown),
// x += alpha p + omega s, r = s - omega t; partials rhat.r and r.r.
template <typename T, typename IT>
__global__ __launch_bounds__(kBlock) void bicg_update_kernel(const IterArgs<T, IT> *__restrict__ A) {
    SolveState *st = A->st;
    if (load_done(st)) return;
    const int it = st->iter_c;
    double tot[3];
    {
        const int slot[3] = {kBiTS, kBiTT, kBiSS};
        load_totals<3>(A->part, gridDim.x, slot, tot);
    }
    const double bb = st->bb;
    const bool half = sqrt(tot[2]) <= A->tol * sqrt(bb);
    if (!half && (tot[1] == 0.0 || tot[0] == 0.0)) {
        if (block0()) st->spmv += 1;
        finish(st, SLA_BREAKDOWN, it, 0.0);
        return;
    }
    const T alpha = (T)st->alpha[it & 1];
    const double omega_d = half ? 0.0 : tot[0] / tot[1];
    const T omega = (T)omega_d;
    const T *__restrict__ p = A->p[(it + 1) & 1];
    const T *__restrict__ s = A->s;
    const T *__restrict__ tv = A->t;
    const T *__restrict__ rh = A->rh;
    T *__restrict__ x = A->x;
    T *__restrict__ r = A->r;
    const int64_t n = A->n;
    double rhr = 0.0, rr = 0.0;
    const TileRange tr = xcd_tiles(tiles_of(n));
    for (int64_t t = tr.first; t < tr.end; t += tr.stride) {
        const int64_t i = t * kTileRows + threadIdx.x;
        if (i < n) {
            if (half) {
                x[i] = fmaB(alpha, p[i], x[i]);
            } else {
                const T si = s[i];
                x[i] = fmaB(omega, si, fmaB(alpha, p[i], x[i]));
                const T ri = fmaB(-omega, tv[i], si);
                r[i] = ri;
                rhr += (double)rh[i] * (double)ri;
                rr += (double)ri * (double)ri;
            }
        }
    }
    if (half) {
        // stop in the next kernel: a block still to start must not see
        // `done` before it has applied its x update
        if (block0()) {
            st->half_ss = tot[2];
            st->half_exit = 1;
            st->iter_a = it + 1;
        }
        return;
    }
    if (block0()) {
        st->omega[it & 1] = omega_d;
        st->iter_a = it + 1;
        st->spmv += 1;
    }
    double v[2] = {rhr, rr};
    const int slot[2] = {kBiRHR, kBiRR};
    store_partials<2>(v, A->part, slot);
}

// ------------------------------------------------------------------ launchers

template <typename T, typename IT>
hipError_t launch_bicg_init(const IterArgs<T, IT> *a, int64_t n, hipStream_t s) {
    bicg_init_kernel<T, IT><<<grid_for_tiles(tiles_of(n)), kBlock, 0, s>>>(a);
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_bicg_pv(int, const IterArgs<T, IT> *a, int64_t n, hipStream_t s) {
    bicg_pv_kernel<T, IT><<<grid_for_tiles(tiles_of(n)), kBlock, 0, s>>>(a);
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_bicg_st(int, const IterArgs<T, IT> *a, int64_t n, hipStream_t s) {
    bicg_st_kernel<T, IT><<<grid_for_tiles(tiles_of(n)), kBlock, 0, s>>>(a);
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_bicg_update(const IterArgs<T, IT> *a, int64_t n, hipStream_t s) {
    bicg_update_kernel<T, IT><<<grid_for_tiles(tiles_of(n)), kBlock, 0, s>>>(a);
    return hipGetLastError();
}

#define SLA_INST(T, IT)                                                                        \
    template hipError_t launch_bicg_init<T, IT>(const IterArgs<T, IT> *, int64_t, hipStream_t); \
    template hipError_t launch_bicg_pv<T, IT>(int, const IterArgs<T, IT> *, int64_t,           \
                                              hipStream_t);                                    \
    template hipError_t launch_bicg_st<T, IT>(int, const IterArgs<T, IT> *, int64_t,           \
                                              hipStream_t);                                    \
    template hipError_t launch_bicg_update<T, IT>(const IterArgs<T, IT> *, int64_t, hipStream_t);

SLA_INST(float, int32_t)
SLA_INST(float, int64_t)
SLA_INST(double, int32_t)
SLA_INST(double, int64_t)

}  // namespace sla
