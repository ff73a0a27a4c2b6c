// BiCGStab for nonsymmetric systems (torch-sla explainer, Methodology
// section 1 lists BiCGStab among the iterative solvers; steps of van der
// Vorst, SIAM J. Sci. Stat. Comput. 13, 1992), unpreconditioned, grid path.
//
// Iteration k, three kernels:
//   bicg_pv:     p = r + beta (p - omega v) evaluated while gathering,
//                v = A p, stored p and v, partial rhat.v
//                -> last block: alpha = rho / rhat.v (0: breakdown)
//   bicg_st:     s = r - alpha v evaluated while gathering, t = A s, stored
//                s and t, partials t.s, t.t, s.s
//                -> last block: half-step test ||s|| <= tol ||b||, else
//                   omega = t.s / t.t (t.t = 0 or t.s = 0: breakdown)
//   bicg_update: half step: x += alpha p; else x += alpha p + omega s,
//                r = s - omega t, partials rhat.r and r.r
//                -> last block: stop test, maxit, next rho and beta
// p and v are double-buffered by iteration parity (the SpMV kernels read the
// old vectors at neighbouring rows while they write the new ones).
#include "sla_internal.h"

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

template <typename T, typename IT>
__global__ __launch_bounds__(kBlock) void bicg_init_kernel(const IterArgs<T, IT> *__restrict__ A) {
    SolveState *st = A->st;
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
    double v[2] = {rr, bb}, tot[2];
    if (grid_reduce<2>(v, A->part, &st->ticket, tot) && threadIdx.x == 0) {
        st->rho = tot[0];  // rhat = r
        st->rr = tot[0];
        st->bb = tot[1];
        st->iter = 0;
        st->alpha = 1.0;
        st->omega = 1.0;
        st->beta = 0.0;
        st->half = 0;
        if (tot[1] == 0.0) {
            st->done = 1;
            st->status = SLA_OK;
            st->zero_x = x0 ? 1 : 0;
        } else if (sqrt(tot[0]) <= A->tol * sqrt(tot[1])) {
            st->done = 1;
            st->status = SLA_OK;
        } else if (A->maxit <= 0) {
            st->done = 1;
            st->status = SLA_NOT_CONVERGED;
        }
    }
}

template <int G, typename T, typename IT>
__global__ __launch_bounds__(kBlock) void bicg_pv_kernel(const IterArgs<T, IT> *__restrict__ A) {
    SolveState *st = A->st;
    if (st->done) return;
    const int it = st->iter;
    const bool first = (it == 0);
    const T beta = (T)st->beta, omega = (T)st->omega;
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
    constexpr int RPP = kBlock / G;
    const int lane = threadIdx.x & (G - 1);
    const int grp = threadIdx.x / G;
    double rv = 0.0;
    const TileRange tr = xcd_tiles(tiles_of(n));
    for (int64_t t = tr.first; t < tr.end; t += tr.stride) {
        const int64_t base = t * kTileRows;
        for (int pass = 0; pass < G; ++pass) {
            const int64_t i = base + pass * RPP + grp;
            if (i < n) {
                const IT e = rp[i + 1];
                T acc = T(0);
                if (first) {
                    for (IT k = rp[i] + lane; k < e; k += G) acc += val[k] * r[col[k]];
                } else {
                    for (IT k = rp[i] + lane; k < e; k += G) {
                        const int32_t c = col[k];
                        acc += val[k] * pdir(false, beta, omega, r[c], pold[c], vold[c]);
                    }
                }
                acc = group_sum<G>(acc);
                if (lane == 0) {
                    pnew[i] = first ? r[i] : pdir(false, beta, omega, r[i], pold[i], vold[i]);
                    vnew[i] = acc;
                    rv += (double)rh[i] * (double)acc;
                }
            }
        }
    }
    double v[1] = {rv}, tot[1];
    if (grid_reduce<1>(v, A->part, &st->ticket, tot) && threadIdx.x == 0) {
        st->aux = tot[0];
        st->spmv += 1;
        st->nfused += 1;
        if (tot[0] == 0.0) {
            st->done = 1;
            st->status = SLA_BREAKDOWN;
        } else {
            st->alpha = st->rho / tot[0];
        }
    }
}

template <int G, typename T, typename IT>
__global__ __launch_bounds__(kBlock) void bicg_st_kernel(const IterArgs<T, IT> *__restrict__ A) {
    SolveState *st = A->st;
    if (st->done) return;
    const int it = st->iter;
    const T alpha = (T)st->alpha;
    const T *__restrict__ r = A->r;
    const T *__restrict__ v = A->v[(it + 1) & 1];
    T *__restrict__ s = A->s;
    T *__restrict__ tv = A->t;
    const IT *__restrict__ rp = A->rp;
    const int32_t *__restrict__ col = A->col;
    const T *__restrict__ val = A->val;
    const int64_t n = A->n;
    constexpr int RPP = kBlock / G;
    const int lane = threadIdx.x & (G - 1);
    const int grp = threadIdx.x / G;
    double ts = 0.0, tt = 0.0, ss = 0.0;
    const TileRange tr = xcd_tiles(tiles_of(n));
    for (int64_t t = tr.first; t < tr.end; t += tr.stride) {
        const int64_t base = t * kTileRows;
        for (int pass = 0; pass < G; ++pass) {
            const int64_t i = base + pass * RPP + grp;
            if (i < n) {
                const IT e = rp[i + 1];
                T acc = T(0);
                for (IT k = rp[i] + lane; k < e; k += G) {
                    const int32_t c = col[k];
                    acc += val[k] * fmaB(-alpha, v[c], r[c]);
                }
                acc = group_sum<G>(acc);
                if (lane == 0) {
                    const T si = fmaB(-alpha, v[i], r[i]);
                    s[i] = si;
                    tv[i] = acc;
                    ts += (double)acc * (double)si;
                    tt += (double)acc * (double)acc;
                    ss += (double)si * (double)si;
                }
            }
        }
    }
    double red[3] = {ts, tt, ss}, tot[3];
    if (grid_reduce<3>(red, A->part, &st->ticket, tot) && threadIdx.x == 0) {
        st->ss = tot[2];
        st->nfused += 1;
        if (sqrt(tot[2]) <= A->tol * sqrt(st->bb)) {
            st->half = 1;  // bicg_update applies x += alpha p and stops
        } else {
            st->spmv += 1;
            if (tot[1] == 0.0 || tot[0] == 0.0) {
                st->done = 1;
                st->status = SLA_BREAKDOWN;
            } else {
                st->omega = tot[0] / tot[1];
            }
        }
    }
}

template <typename T, typename IT>
__global__ __launch_bounds__(kBlock) void bicg_update_kernel(const IterArgs<T, IT> *__restrict__ A) {
    SolveState *st = A->st;
    if (st->done) return;
    const int it = st->iter;
    const bool half = st->half != 0;
    const T alpha = (T)st->alpha, omega = (T)st->omega;
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
    double v[2] = {rhr, rr}, tot[2];
    if (grid_reduce<2>(v, A->part, &st->ticket, tot) && threadIdx.x == 0) {
        const int k = it + 1;
        st->iter = k;
        if (half) {
            st->rr = st->ss;
            st->done = 1;
            st->status = SLA_OK;
        } else {
            st->rr = tot[1];
            if (sqrt(tot[1]) <= A->tol * sqrt(st->bb)) {
                st->done = 1;
                st->status = SLA_OK;
            } else if (k >= A->maxit) {
                st->done = 1;
                st->status = SLA_NOT_CONVERGED;
            } else if (tot[0] == 0.0) {
                st->done = 1;
                st->status = SLA_BREAKDOWN;
            } else {
                st->beta = (tot[0] / st->rho) * (st->alpha / st->omega);
                st->rho = tot[0];
            }
        }
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
hipError_t launch_bicg_init(const IterArgs<T, IT> *a, int64_t n, hipStream_t s) {
    bicg_init_kernel<T, IT><<<grid_for_tiles(tiles_of(n)), kBlock, 0, s>>>(a);
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_bicg_pv(int G, const IterArgs<T, IT> *a, int64_t n, hipStream_t s) {
    const int grid = grid_for_tiles(tiles_of(n));
    SLA_DISPATCH_G(G, bicg_pv_kernel<kG, T, IT><<<grid, kBlock, 0, s>>>(a));
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_bicg_st(int G, const IterArgs<T, IT> *a, int64_t n, hipStream_t s) {
    const int grid = grid_for_tiles(tiles_of(n));
    SLA_DISPATCH_G(G, bicg_st_kernel<kG, T, IT><<<grid, kBlock, 0, s>>>(a));
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
