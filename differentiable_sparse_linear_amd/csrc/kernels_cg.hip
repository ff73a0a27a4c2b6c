// Conjugate gradients with an optional Jacobi preconditioner M = diag(A)
// (torch-sla explainer, Methodology section 1 and the Significance section:
// the native backend is an iterative solver with a Jacobi preconditioner).
//
// Grid path: the Chronopoulos-Gear arrangement of preconditioned CG, which
// produces the same iterates as the textbook recurrence (Saad, Iterative
// Methods for Sparse Linear Systems, Alg. 9.1) in exact arithmetic but needs
// one global reduction per iteration instead of two:
//   r_0 = b - A x_0, u_0 = M^-1 r_0, w_0 = A u_0
//   iteration i: gamma_i = r_i.u_i, delta_i = w_i.u_i
//     beta_i  = gamma_i / gamma_{i-1}                       (beta_0 = 0)
//     alpha_i = gamma_i / (delta_i - beta_i gamma_i / alpha_{i-1})
//             = gamma_i / (p_i . A p_i)                     (<= 0: breakdown)
//     p_i = u_i + beta_i p_{i-1},  s_i = w_i + beta_i s_{i-1}  (= A p_i)
//     x_{i+1} = x_i + alpha_i p_i,  r_{i+1} = r_i - alpha_i s_i
//     u_{i+1} = M^-1 r_{i+1},  w_{i+1} = A u_{i+1}
// One kernel does a whole iteration: the vector updates of its rows, and the
// product w_{i+1} = A u_{i+1} with u_{i+1} evaluated at each gathered column
// from r_i, w_i, s_{i-1} and M^-1.  It stores per-block partial sums of
// gamma_{i+1}, delta_{i+1} and ||r_{i+1}||^2 with plain stores; every block
// of the next launch adds them in block order (identical scalars everywhere,
// no grid-wide fence).  r, w, s and the partial-sum slots alternate between
// two buffers by iteration parity, which each launch receives as an argument
// (neighbouring rows still read the old vectors while a block writes the new
// ones).  Every launch returns at entry once the device-side `done` flag is
// set, so the host enqueues many iterations (HIP graph replays) and polls
// rarely.
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

// Vectors of the grid CG in the workspace: r by parity = {r, z}, w = {q, rh},
// s = {s, t}, p = p[0]; t doubles as A x0 before the first iteration.
// (Selected with conditionals: a pointer array indexed by a runtime parity
// would live in scratch memory.)
template <typename T, typename IT>
__device__ __forceinline__ T *cg_r(const IterArgs<T, IT> *A, int ph) { return ph ? A->z : A->r; }
template <typename T, typename IT>
__device__ __forceinline__ T *cg_w(const IterArgs<T, IT> *A, int ph) { return ph ? A->rh : A->q; }
template <typename T, typename IT>
__device__ __forceinline__ T *cg_s(const IterArgs<T, IT> *A, int ph) { return ph ? A->t : A->s; }

template <typename T>
struct CgOwn {
    T r, w, s, d, p, x;
};

// r_0 = b - A x_0, u_0 = M^-1 r_0, w_0 = A u_0 (A x_0 is in t; the host
// zeroes t when there is no initial guess); partials gamma_0, delta_0,
// ||r_0||^2 and ||b||^2 (parity-0 slots).
template <typename T, typename IT, bool JAC, int SLOTS>
__global__ __launch_bounds__(kBlock) void cg_init_kernel(const IterArgs<T, IT> *__restrict__ A) {
    const int64_t n = A->n;
    const gptr<const T> b = glb(A->b);
    const gptr<const T> ax0 = glb((const T *)cg_s(A, 1));
    const gptr<const T> dinv = glb(A->dinv);
    const gptr<const T> val = glb(A->val);
    const gptr<T> x = glb(A->x);
    const gptr<T> r0 = glb(cg_r(A, 0));
    const gptr<T> w0 = glb(cg_w(A, 0));
    const bool x0 = A->use_x0 != 0;
    __shared__ SpmvLds<T, IT> sm;
    double ga = 0.0, de = 0.0, rr = 0.0, bb = 0.0;
    auto load = [&](int64_t c) { return G3<T>{b[c], ax0[c], JAC ? dinv[c] : T(1)}; };
    auto u0 = [&](const G3<T> &g) -> T { return JAC ? g.c * (g.a - g.b) : g.a - g.b; };
    SLA_SPMV_LOOP<T, IT, SLOTS, SLOTS>(
        xcd_tiles(tiles_of(n)), n, glb(A->rp), glb(A->col), sm, [&](IT k) { return val[k]; },
        load, u0, load,
        [&](int64_t i, T acc, const G3<T> &o) {
            const T ri = o.a - o.b;
            const T ui = u0(o);
            r0[i] = ri;
            w0[i] = acc;
            if (!x0) x[i] = T(0);
            ga += (double)ri * (double)ui;
            de += (double)acc * (double)ui;
            rr += (double)ri * (double)ri;
            bb += (double)o.a * (double)o.a;
        },
        NoPre(), NoPost());
    double v[4] = {ga, de, rr, bb};
    const int slot[4] = {kCgGA, kCgDE, kCgRR, kCgBB};
    store_partials<4>(v, A->part, slot);
}

// Iteration i (i = st->iter_p[ph], ph = i & 1): stop tests on r_i, the
// scalars, the row updates and w_{i+1} = A u_{i+1}.
#ifndef SLA_CG_ROUND
#define SLA_CG_ROUND 4
#endif
template <typename T, typename IT, bool JAC, int SLOTS>
__global__ __launch_bounds__(kBlock) void cg_iter_kernel(const IterArgs<T, IT> *__restrict__ A,
                                                         int ph) {
    SolveState *st = A->st;
    if (load_done(st)) return;
    const int it = st->iter_p[ph];
    const bool first = (it == 0);
    const int64_t n = A->n;
    const gptr<const T> val = glb(A->val);
    const gptr<const T> dinv = glb(A->dinv);
    const gptr<const T> rc = glb((const T *)cg_r(A, ph));
    const gptr<const T> wc = glb((const T *)cg_w(A, ph));
    const gptr<const T> sp = glb((const T *)cg_s(A, ph ^ 1));
    const gptr<T> rn = glb(cg_r(A, ph ^ 1));
    const gptr<T> wn = glb(cg_w(A, ph ^ 1));
    const gptr<T> sc = glb(cg_s(A, ph));
    const gptr<T> p = glb(A->p[0]);
    const gptr<T> x = glb(A->x);
    __shared__ SpmvLds<T, IT> sm;
    __shared__ double red[4][kWaves];

    // previous launch's partial sums, loaded with the first row pointers
    auto pre = [&]() {
        if (it == 0) {
            const int slot[4] = {kCgGA, kCgDE, kCgRR, kCgBB};
            partial_loads<4>(A->part, slot, red);
        } else {
            const int slot[3] = {ph ? kCgGA1 : kCgGA, ph ? kCgDE1 : kCgDE, ph ? kCgRR1 : kCgRR};
            partial_loads<3>(A->part, slot, red);
        }
    };
    T beta = T(0), alpha = T(0);
    auto post = [&]() -> bool {
        double tot[4];
        if (it == 0) {
            totals<4>(red, tot);
        } else {
            double t3[3];
            totals<3>(red, t3);
            tot[0] = t3[0];
            tot[1] = t3[1];
            tot[2] = t3[2];
            tot[3] = st->bb;
        }
        const double gamma = tot[0], delta = tot[1], rr = tot[2], bb = tot[3];
        if (it == 0 && st->zero_diag) {
            finish(st, SLA_ERR_ZERO_DIAG, 0, rr);
            return false;
        }
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
        const double beta_d = first ? 0.0 : gamma / st->rho[ph ^ 1];
        const double den = first ? delta : delta - beta_d * gamma / st->alpha[ph ^ 1];
        if (!(den > 0.0)) {
            finish(st, SLA_BREAKDOWN, it, rr);
            return false;
        }
        const double alpha_d = gamma / den;
        if (block0()) {
            st->rho[ph] = gamma;
            st->alpha[ph] = alpha_d;
            st->iter_p[ph ^ 1] = it + 1;
            st->nfused += 1;
            st->spmv += first ? (A->use_x0 ? 3 : 2) : 1;  // init (and A x0) products
            if (first) st->bb = bb;
        }
        beta = (T)beta_d;
        alpha = (T)alpha_d;
        return true;
    };
    // s_i and u_{i+1} from the four vectors at one index (the gathers and the
    // row updates use the same expressions, so they see the same values).
    // The first iteration has beta = 0 and reads w and r in place of the
    // (not yet written) previous s and p: fma(0, finite, w) == w exactly.
    const gptr<const T> sprev = first ? wc : sp;
    const gptr<const T> pprev = first ? rc : (gptr<const T>)p;
    auto s_of = [&](T w, T sv) -> T { return fmaT(beta, sv, w); };
    auto u_of = [&](const G4<T> &g) -> T {
        const T rv = fmaT(-alpha, s_of(g.b, g.c), g.a);
        return JAC ? g.d * rv : rv;
    };
    double g = 0.0, d = 0.0, q = 0.0;
    const bool go = SLA_SPMV_LOOP<T, IT, SLOTS, SLA_CG_ROUND>(
        xcd_tiles(tiles_of(n)), n, glb(A->rp), glb(A->col), sm, [&](IT k) { return val[k]; },
        [&](int32_t c) { return G4<T>{rc[c], wc[c], sprev[c], JAC ? dinv[c] : T(1)}; }, u_of,
        [&](int64_t i) { return CgOwn<T>{rc[i], wc[i], sprev[i], JAC ? dinv[i] : T(1), pprev[i], x[i]}; },
        [&](int64_t i, T acc, const CgOwn<T> &o) {
            const T ui = JAC ? o.d * o.r : o.r;
            const T pi = fmaT(beta, o.p, ui);
            const T si = s_of(o.w, o.s);
            const T rni = fmaT(-alpha, si, o.r);
            const T uni = JAC ? o.d * rni : rni;
            x[i] = fmaT(alpha, pi, o.x);
            p[i] = pi;
            sc[i] = si;
            rn[i] = rni;
            wn[i] = acc;
            g += (double)rni * (double)uni;
            d += (double)acc * (double)uni;
            q += (double)rni * (double)rni;
        },
        pre, post);
    if (!go) return;
    double v[3] = {g, d, q};
    const int slot[3] = {ph ? kCgGA : kCgGA1, ph ? kCgDE : kCgDE1, ph ? kCgRR : kCgRR1};
    store_partials<3>(v, A->part, slot);
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
hipError_t launch_cg_init(int slots, bool jac, const IterArgs<T, IT> *a, int64_t n, hipStream_t s) {
    const int grid = grid_for_tiles(tiles_of(n));
    if (jac) {
        SLA_DISPATCH_SLOTS(slots, cg_init_kernel<T, IT, true, kS><<<grid, kBlock, 0, s>>>(a));
    } else {
        SLA_DISPATCH_SLOTS(slots, cg_init_kernel<T, IT, false, kS><<<grid, kBlock, 0, s>>>(a));
    }
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_cg_iter(int slots, bool jac, const IterArgs<T, IT> *a, int64_t n, int ph,
                          hipStream_t s) {
    const int grid = grid_for_tiles(tiles_of(n));
    if (jac) {
        SLA_DISPATCH_SLOTS(slots, cg_iter_kernel<T, IT, true, kS><<<grid, kBlock, 0, s>>>(a, ph));
    } else {
        SLA_DISPATCH_SLOTS(slots, cg_iter_kernel<T, IT, false, kS><<<grid, kBlock, 0, s>>>(a, ph));
    }
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
    template hipError_t launch_cg_init<T, IT>(int, bool, const IterArgs<T, IT> *, int64_t,      \
                                              hipStream_t);                                     \
    template hipError_t launch_cg_iter<T, IT>(int, bool, const IterArgs<T, IT> *, int64_t, int, \
                                              hipStream_t);                                     \
    template hipError_t launch_block_cg<T, IT>(int, const BlockCgParams &, int, hipStream_t);

SLA_INST(float, int32_t)
SLA_INST(float, int64_t)
SLA_INST(double, int32_t)
SLA_INST(double, int64_t)

}  // namespace sla
