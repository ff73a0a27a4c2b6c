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
    const gptr<const T> b = glb(A->b);
    const gptr<const T> ax0 = glb((const T *)A->q);
    const gptr<T> x = glb(A->x);
    const gptr<T> r = glb(A->r);
    const gptr<T> rh = glb(A->rh);
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

template <typename T>
struct PvOwn {
    T r, p, v, rh;
};

// Iteration k (0-based, k = iter_a): a pending half-step exit stops here;
// stop tests on r_k; rho_k = rhat.r_k (0: breakdown);
// beta = (rho_k/rho_{k-1})(alpha_{k-1}/omega_{k-1});
// p = r + beta (p - omega v) evaluated while gathering (p = r at k = 0);
// v = A p; partial rhat.v.
#ifndef SLA_BICG_WAVES
#define SLA_BICG_WAVES 5
#endif
template <typename T, typename IT, int SLOTS, int CM>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(CM == kColDiaMajor ? 4 : SLA_BICG_WAVES)))
void bicg_pv_kernel(const IterArgs<T, IT> *__restrict__ A) {
    SolveState *st = A->st;
    if (load_done(st)) return;
    const int it = st->iter_a;
    const bool first = (it == 0);
    const int64_t n = A->n;
    const gptr<const T> val = glb(A->val);
    const gptr<const T> r = glb((const T *)A->r);
    const gptr<const T> rh = glb((const T *)A->rh);
    const gptr<const T> pold = glb((const T *)A->p[it & 1]);
    const gptr<const T> vold = glb((const T *)A->v[it & 1]);
    const gptr<T> pnew = glb(A->p[(it + 1) & 1]);
    const gptr<T> vnew = glb(A->v[(it + 1) & 1]);
    __shared__ RowLds<T, IT> sm;
    __shared__ double red[3][kWaves];
    auto pre = [&]() {
        const int slot[3] = {kBiRHR, kBiRR, kBiBB};
        partial_loads<3>(A->part, slot, red);
    };
    T beta = T(0), omega = T(0);
    auto post = [&]() -> bool {
        if (st->half_exit) {
            finish(st, SLA_OK, it, st->half_ss);
            return false;
        }
        double tot[3];
        totals<3>(red, tot);
        const double rho = tot[0], rr = tot[1];
        const double bb = it == 0 ? tot[2] : st->bb;
        if (it == 0 && bb == 0.0) {
            if (block0()) st->zero_x = A->use_x0 ? 1 : 0;
            finish(st, SLA_OK, 0, 0.0);
            return false;
        }
        if (sqrt(rr) <= A->tol * sqrt(bb)) {
            finish(st, SLA_OK, it, rr);
            return false;
        }
        if (it >= A->maxit) {
            finish(st, SLA_NOT_CONVERGED, it, rr);
            return false;
        }
        if (rho == 0.0) {
            finish(st, SLA_BREAKDOWN, it, rr);
            return false;
        }
        const int pv = (it + 1) & 1;  // parity slot of iteration k-1
        beta = first ? T(0) : (T)((rho / st->rho[pv]) * (st->alpha[pv] / st->omega[pv]));
        omega = first ? T(0) : (T)st->omega[pv];
        if (block0()) {
            st->rho[it & 1] = rho;
            st->iter_b = it;
            st->spmv += (first && A->use_x0) ? 2 : 1;  // counts the A x0 product
            st->nfused += 1;
            if (first) st->bb = bb;
        }
        return true;
    };
    // p_k at one index; the first iteration has beta = omega = 0 and reads r
    // in place of the (not yet written) previous p and v, which gives r
    // exactly
    const gptr<const T> pp = first ? r : pold;
    const gptr<const T> vp = first ? r : vold;
    auto pk = [&](const G3<T> &g) -> T { return pdir(false, beta, omega, g.a, g.b, g.c); };
    double rv_acc = 0.0;
    const bool go = spmv_rows<T, IT, SLOTS, 4>(
        xcd_tiles(tiles_of(n)), n, glb(A->rp), col_src<CM>(A->cols), sm, [&](auto k) { return val[k]; },
        [&](int32_t c) { return G3<T>{r[c], pp[c], vp[c]}; }, pk,
        [&](int64_t i) { return PvOwn<T>{r[i], pp[i], vp[i], rh[i]}; },
        [&](int64_t i, T acc, const PvOwn<T> &o, T) {
            pnew[i] = pk(G3<T>{o.r, o.p, o.v});
            vnew[i] = acc;
            rv_acc += (double)o.rh * (double)acc;
        },
        pre, post);
    if (!go) return;
    double v[1] = {rv_acc};
    const int slot[1] = {kBiRV};
    store_partials<1>(v, A->part, slot);
}

template <typename T>
struct StOwn {
    T r, v;
};

// Iteration k (k = iter_b): alpha = rho_k / rhat.v (0: breakdown);
// s = r - alpha v evaluated while gathering, t = A s; partials t.s, t.t, s.s.
template <typename T, typename IT, int SLOTS, int CM>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(CM == kColDiaMajor ? 4 : SLA_BICG_WAVES)))
void bicg_st_kernel(const IterArgs<T, IT> *__restrict__ A) {
    SolveState *st = A->st;
    if (load_done(st)) return;
    const int it = st->iter_b;
    const int64_t n = A->n;
    const gptr<const T> val = glb(A->val);
    const gptr<const T> r = glb((const T *)A->r);
    const gptr<const T> v = glb((const T *)A->v[(it + 1) & 1]);
    const gptr<T> s = glb(A->s);
    const gptr<T> tv = glb(A->t);
    __shared__ RowLds<T, IT> sm;
    __shared__ double red[1][kWaves];
    auto pre = [&]() {
        const int slot[1] = {kBiRV};
        partial_loads<1>(A->part, slot, red);
    };
    T alpha = T(0);
    auto post = [&]() -> bool {
        double tot[1];
        totals<1>(red, tot);
        if (tot[0] == 0.0) {
            finish(st, SLA_BREAKDOWN, it, 0.0);
            return false;
        }
        const double alpha_d = st->rho[it & 1] / tot[0];
        alpha = (T)alpha_d;
        if (block0()) {
            st->alpha[it & 1] = alpha_d;
            st->iter_c = it;
            st->nfused += 1;
        }
        return true;
    };
    auto sk = [&](const G2<T> &g) -> T { return fmaB(-alpha, g.b, g.a); };
    double ts = 0.0, tt = 0.0, ss = 0.0;
    const bool go = spmv_rows<T, IT, SLOTS, SLOTS>(
        xcd_tiles(tiles_of(n)), n, glb(A->rp), col_src<CM>(A->cols), sm, [&](auto k) { return val[k]; },
        [&](int32_t c) { return G2<T>{r[c], v[c]}; }, sk,
        [&](int64_t i) { return StOwn<T>{r[i], v[i]}; },
        [&](int64_t i, T acc, const StOwn<T> &o, T) {
            const T si = sk(G2<T>{o.r, o.v});
            s[i] = si;
            tv[i] = acc;
            ts += (double)acc * (double)si;
            tt += (double)acc * (double)acc;
            ss += (double)si * (double)si;
        },
        pre, post);
    if (!go) return;
    double red3[3] = {ts, tt, ss};
    const int slot[3] = {kBiTS, kBiTT, kBiSS};
    store_partials<3>(red3, A->part, slot);
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
    const gptr<const T> p = glb((const T *)A->p[(it + 1) & 1]);
    const gptr<const T> s = glb((const T *)A->s);
    const gptr<const T> tv = glb((const T *)A->t);
    const gptr<const T> rh = glb((const T *)A->rh);
    const gptr<T> x = glb(A->x);
    const gptr<T> r = glb(A->r);
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
hipError_t launch_bicg_pv(int slots, int cm, const IterArgs<T, IT> *a, int64_t n,
                          hipStream_t s, const hipEvent_t *ev) {
    const dim3 grid(grid_for_tiles(tiles_of(n)));
    SLA_DISPATCH_FORM(cm, slots, launch_maybe_timed(
                                                        bicg_pv_kernel<T, IT, kS, kC>, grid,
                                                        dim3(kBlock), 0, s, ev, a));
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_bicg_st(int slots, int cm, const IterArgs<T, IT> *a, int64_t n,
                          hipStream_t s, const hipEvent_t *ev) {
    const dim3 grid(grid_for_tiles(tiles_of(n)));
    SLA_DISPATCH_FORM(cm, slots, launch_maybe_timed(
                                                        bicg_st_kernel<T, IT, kS, kC>, grid,
                                                        dim3(kBlock), 0, s, ev, a));
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_bicg_update(const IterArgs<T, IT> *a, int64_t n, hipStream_t s) {
    bicg_update_kernel<T, IT><<<grid_for_tiles(tiles_of(n)), kBlock, 0, s>>>(a);
    return hipGetLastError();
}

#define SLA_INST(T, IT)                                                                        \
    template hipError_t launch_bicg_init<T, IT>(const IterArgs<T, IT> *, int64_t, hipStream_t); \
    template hipError_t launch_bicg_pv<T, IT>(int, int, const IterArgs<T, IT> *, int64_t,     \
                                              hipStream_t, const hipEvent_t *);                \
    template hipError_t launch_bicg_st<T, IT>(int, int, const IterArgs<T, IT> *, int64_t,     \
                                              hipStream_t, const hipEvent_t *);                \
    template hipError_t launch_bicg_update<T, IT>(const IterArgs<T, IT> *, int64_t, hipStream_t);

SLA_INST(float, int32_t)
SLA_INST(float, int64_t)
SLA_INST(double, int32_t)
SLA_INST(double, int64_t)

}  // namespace sla
