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
// With M = diag(A) the kernels keep the scaled vectors u = M^-1 r,
// w^ = M^-1 w and s^ = M^-1 s instead of r, w and s: then
//   s^_i = w^_i + beta_i s^_{i-1},  u_{i+1} = u_i - alpha_i s^_i,
//   w^_{i+1} = (A u_{i+1}) / a_ii,  r = a_ii u,
// so the product's gathers need u, w^ and s^ only (no M^-1 vector) and a_ii
// comes from the row's own diagonal entry.  Without a preconditioner a_ii is
// taken as 1 and the same code runs on r, w and s.
// One kernel does a whole iteration: the vector updates of its rows, and the
// product w_{i+1} = A u_{i+1} with u_{i+1} evaluated at each gathered column
// from u_i, w^_i and s^_{i-1}.  It stores per-block partial sums of
// gamma_{i+1}, delta_{i+1} and ||r_{i+1}||^2 with plain stores; every block
// of the next launch adds them in block order (identical scalars everywhere,
// no grid-wide fence).  u, w^, s^ and the partial-sum slots alternate between
// two buffers by iteration parity, a template argument of the kernel
// (neighbouring rows still read the old vectors while a block writes the new
// ones).  x is brought up to date every second iteration: the odd launch i
// adds alpha_{i-1} p_{i-1} + alpha_i p_i (p_{i-1} is read anyway); a stop at
// an odd iteration leaves x one step behind and flags it, and one launch
// after the solve adds the pending alpha_{i-1} p_{i-1} (in the stopping launch
// itself, blocks that start after block 0 has set `done` would skip it).
// Once the device-side `done` flag is set every launch ends at its first
// barrier without loading anything (each wavefront reads the flag at entry;
// the block acts on what its wavefronts saw together, so they cannot split),
// so the host enqueues many iterations (HIP graph replays) and polls rarely.
// A launch may advance several systems of a batch (blockIdx.y is the
// system, whose own argument block points at its vectors, state and partial
// sums, so the kernel body is that of one system); a system that
// has stopped ends at the first barrier while the others go on, and the host waits
// for the count of stopped systems.  The one-workgroup solver for systems of
// at most 4096 rows is in kernels_block.hip.
#include "spmv_tile.h"

namespace sla {

template <typename T>
__device__ __forceinline__ T fmaT(T a, T b, T c) {
    return fma(a, b, c);
}

// Vectors of the grid CG in the workspace: u by parity = {r, z}, w^ = {q, rh},
// s^ = {s, t}, p = p[0]; t doubles as A x0 before the first iteration.
// (Selected with conditionals: a pointer array indexed by a runtime parity
// would live in scratch memory.)
template <typename T, typename IT>
__device__ __forceinline__ T *cg_u(const IterArgs<T, IT> *A, int ph) { return ph ? A->z : A->r; }
template <typename T, typename IT>
__device__ __forceinline__ T *cg_w(const IterArgs<T, IT> *A, int ph) { return ph ? A->rh : A->q; }
template <typename T, typename IT>
__device__ __forceinline__ T *cg_s(const IterArgs<T, IT> *A, int ph) { return ph ? A->t : A->s; }

template <typename T>
struct CgOwn {
    T u, w, s, p, x;
};

// The column source of the iterations: a diagonal-major operator whose
// offsets mirror reads its lower diagonals through their mirrors unless the
// pack found the system's values unsymmetric.
template <int CM>
__device__ __forceinline__ ColSrc<CM> cg_cols(const ColArgs &a, const SolveState *st) {
    ColSrc<CM> c = col_src<CM>(a);
    if constexpr (CM == kColDiaMajor) c.sym = c.sym && !st->asym;
    return c;
}

// r_0 = b - A x_0 (A x_0 is in t; the host zeroes t when there is no initial
// guess), u_0 = M^-1 r_0, w_0 = A u_0; stores u_0 and w^_0 = M^-1 w_0 in the
// parity-0 buffers and zeroes x without an initial guess; partials gamma_0,
// delta_0, ||r_0||^2 and ||b||^2 (parity-0 slots).
template <typename T, typename IT, bool JAC, int SLOTS, int CM>
__global__ __launch_bounds__(kBlock) void cg_init_kernel(const IterArgs<T, IT> *__restrict__ A) {
    A += blockIdx.y;
    const int64_t n = A->n;
    const gptr<const T> b = glb(A->b);
    const gptr<const T> ax0 = glb((const T *)cg_s(A, 1));
    const gptr<const T> dinv = glb(A->dinv);
    const gptr<const T> val = glb(A->val);
    const gptr<T> x = glb(A->x);
    const gptr<T> u0 = glb(cg_u(A, 0));
    const gptr<T> w0 = glb(cg_w(A, 0));
    const bool x0 = A->use_x0 != 0;
    __shared__ RowLds<T, IT> sm;
    double ga = 0.0, de = 0.0, rr = 0.0, bb = 0.0;
    auto load = [&](int64_t c) { return G3<T>{b[c], ax0[c], JAC ? dinv[c] : T(1)}; };
    auto u_of = [&](const G3<T> &g) -> T { return JAC ? g.c * (g.a - g.b) : g.a - g.b; };
    spmv_rows<T, IT, SLOTS, SLOTS, CM, true>(
        xcd_tiles(tiles_of(n)), n, glb(A->rp), cg_cols<CM>(A->cols, A->st), sm,
        [&](auto k) { return val[k]; }, load, u_of, load,
        [&](int64_t i, T acc, const G3<T> &o, T) {
            const T ri = o.a - o.b;
            const T ui = u_of(o);
            u0[i] = ui;
            w0[i] = JAC ? acc * o.c : acc;
            if (!x0) x[i] = T(0);
            ga = fma((double)ri, (double)ui, ga);
            de = fma((double)acc, (double)ui, de);
            rr = fma((double)ri, (double)ri, rr);
            bb = fma((double)o.a, (double)o.a, bb);
        },
        NoPre(), NoPost());
    double v[4] = {ga, de, rr, bb};
    const int slot[4] = {kCgGA, kCgDE, kCgRR, kCgBB};
    store_partials<4>(v, A->part, slot);
}

// Iteration i (i = st->iter_p[PH], PH = i & 1): stop tests on r_i, the
// scalars, the row updates and w_{i+1} = A u_{i+1}.
#ifndef SLA_CG_ROUND
#define SLA_CG_ROUND 4
#endif
#ifndef SLA_CG_WAVES
#define SLA_CG_WAVES 5
#endif
// ZW: 0, or the z-walk of dia_rows_zw (diagonal-major, seven diagonals, a
// plan from cg_zwalk_plan in the operator's column arguments); ZW == 2
// streams the values, p, x and the vectors written here with non-temporal
// hints (grids far beyond the Infinity Cache, where these are touched once
// per iteration and L2 is better left to the plane's +-N neighbours).
// O32: the fast diagonal-major tiles (ZW == 0, dia_tile): 32-bit byte
// offsets (elem) and the +-1 gathers from the adjacent lanes (dia_rows ADJ);
// PAIR: the same with two rows per lane (fp64, dia_rows_pair).
template <typename T, typename IT, bool JAC, int SLOTS, int PH, int CM, int ZW = 0,
          bool O32 = false, bool PAIR = false>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(CM == kColDiaMajor ? (ZW ? 4 : 3) : SLA_CG_WAVES)))
void cg_iter_kernel(const IterArgs<T, IT> *__restrict__ A) {
    static_assert(!ZW || (CM == kColDiaMajor && SLOTS == 7), "the z-walk is for seven diagonals");
    static_assert(!O32 || (CM == kColDiaMajor && !ZW), "32-bit offsets: diagonal-major tiles");
    static_assert(!PAIR || (O32 && sizeof(T) == 8), "row pairs: fast fp64 tiles");
    constexpr bool NT = ZW == 2;
    A += blockIdx.y;
    SolveState *st = A->st;
    __shared__ int seen[kWaves];
    const bool stopped = saw_stop(st, seen);
    const int it = st->iter_p[PH];
    const bool first = PH == 0 && it == 0;
    const int64_t n = A->n;
    double *part = A->part;
    const gptr<const T> val = glb(A->val);
    const gptr<const T> uc = glb((const T *)cg_u(A, PH));
    const gptr<const T> wc = glb((const T *)cg_w(A, PH));
    const gptr<const T> sp = glb((const T *)cg_s(A, PH ^ 1));
    const gptr<T> un = glb(cg_u(A, PH ^ 1));
    const gptr<T> wn = glb(cg_w(A, PH ^ 1));
    const gptr<T> sc = glb(cg_s(A, PH));
    const gptr<T> p = glb(A->p[0]);
    const gptr<T> x = glb(A->x);
    __shared__ RowLds<T, IT> sm;
    __shared__ double red[4][kWaves];

    // previous launch's partial sums, loaded with the first row pointers
    auto pre = [&]() {
        if (stopped) return;
        if (first) {
            const int slot[4] = {kCgGA, kCgDE, kCgRR, kCgBB};
            partial_loads<4>(part, slot, red);
        } else {
            const int slot[3] = {PH ? kCgGA1 : kCgGA, PH ? kCgDE1 : kCgDE, PH ? kCgRR1 : kCgRR};
            partial_loads<3>(part, slot, red);
        }
    };
    T beta = T(0), alpha = T(0), alpha_prev = T(0);
    // a stop at an odd iteration leaves x = x_{i-1}
    auto stop = [&](int status, double rr) {
        if (PH == 1 && block0()) st->lag = 1;
        finish(st, A->ndone, status, it, rr);
    };
    auto post = [&]() -> bool {
        if (any_saw_stop(seen)) return false;
        double tot[4];
        if (first) {
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
        if (PH == 1) alpha_prev = (T)st->alpha[0];
        if (first && st->zero_diag) {
            finish(st, A->ndone, SLA_ERR_ZERO_DIAG, 0, rr);
            return false;
        }
        if (first && bb == 0.0) {
            if (block0()) st->zero_x = A->use_x0 ? 1 : 0;
            finish(st, A->ndone, SLA_OK, 0, 0.0);
            return false;
        }
        if (sqrt(rr) <= A->tol * sqrt(bb)) {
            stop(SLA_OK, rr);
            return false;
        }
        if (it >= A->maxit) {
            stop(SLA_NOT_CONVERGED, rr);
            return false;
        }
        const double beta_d = first ? 0.0 : gamma / st->rho[PH ^ 1];
        const double den = first ? delta : delta - beta_d * gamma / st->alpha[PH ^ 1];
        if (!(den > 0.0)) {
            stop(SLA_BREAKDOWN, rr);
            return false;
        }
        const double alpha_d = gamma / den;
        if (block0()) {
            st->rho[PH] = gamma;
            st->alpha[PH] = alpha_d;
            st->iter_p[PH ^ 1] = it + 1;
            st->nfused += 1;
            st->spmv += first ? (A->use_x0 ? 3 : 2) : 1;  // init (and A x0) products
            if (first) st->bb = bb;
        }
        beta = (T)beta_d;
        alpha = (T)alpha_d;
        return true;
    };
    // s^_i and u_{i+1} from the three vectors at one index (the gathers and
    // the row updates use the same expressions, so they see the same values).
    // The first iteration has beta = 0 and reads w^ and u in place of the
    // (not yet written) previous s^ and p: fma(0, finite, w) == w exactly.
    const gptr<const T> sprev = first ? wc : sp;
    const gptr<const T> pprev = first ? uc : (gptr<const T>)p;
    auto s_of = [&](T w, T sv) -> T { return fmaT(beta, sv, w); };
    auto u_of = [&](const G3<T> &g) -> T { return fmaT(-alpha, s_of(g.b, g.c), g.a); };
    double g = 0.0, d = 0.0, q = 0.0;
    auto ld = [&](gptr<const T> v, int64_t i) -> T { return *elem<O32>(v, i); };
    auto gath = [&](int32_t c) { return G3<T>{ld(uc, c), ld(wc, c), ld(sprev, c)}; };
    auto put = [&](gptr<T> v, int64_t i, T a) {
        if constexpr (NT)
            __builtin_nontemporal_store(a, elem<O32>(v, i));
        else
            *elem<O32>(v, i) = a;
    };
    auto stream = [&](gptr<const T> v, int64_t i) -> T {
        if constexpr (NT)
            return __builtin_nontemporal_load(elem<O32>(v, i));
        else
            return ld(v, i);
    };
    auto row = [&](int64_t i, T acc, const CgOwn<T> &o, T aii) {
        const T pi = fmaT(beta, o.p, o.u);
        const T si = s_of(o.w, o.s);
        const T uni = fmaT(-alpha, si, o.u);
        if (PH) put(x, i, fmaT(alpha, pi, fmaT(alpha_prev, o.p, o.x)));
        put(p, i, pi);
        put(sc, i, si);
        put(un, i, uni);
        put(wn, i, JAC ? acc / aii : acc);
        const T rni = JAC ? aii * uni : uni;
        g = fma((double)rni, (double)uni, g);
        d = fma((double)acc, (double)uni, d);
        q = fma((double)rni, (double)rni, q);
    };
    bool go;
    if constexpr (ZW) {
        __shared__ G3<T> zring[3][kTileRows];
        go = dia_rows_zw<T>(
            !stopped, n, cg_cols<CM>(A->cols, st), [&](auto k) { return stream(val, k); },
            [&](auto k) { return val[k]; }, gath, u_of,
            [&](int64_t i, const G3<T> &o) {
                return CgOwn<T>{o.a, o.b, o.c, stream(pprev, i),
                                PH ? stream((gptr<const T>)x, i) : T(0)};
            },
            row, pre, post, zring);
    } else {
        auto own_of = [&](int64_t i) {
            return CgOwn<T>{ld(uc, i), ld(wc, i), ld(sprev, i), ld(pprev, i),
                            PH ? ld((gptr<const T>)x, i) : T(0)};
        };
        if constexpr (PAIR) {
            auto ld2 = [&](gptr<const T> v, int64_t i) -> pair_t {
                return *(const __attribute__((address_space(1))) pair_t *)elem<O32>(v, i);
            };
            auto put2 = [&](gptr<T> v, int64_t i, pair_t a) {
                *(__attribute__((address_space(1))) pair_t *)elem<O32>(v, i) = a;
            };
            // row's updates and partial-sum terms for rows i and i + 1
            auto row2 = [&](int64_t i, T acc0, T acc1, const CgOwn<pair_t> &o, T a0, T a1) {
                const pair_t pi = {fmaT(beta, o.p.x, o.u.x), fmaT(beta, o.p.y, o.u.y)};
                const pair_t si = {s_of(o.w.x, o.s.x), s_of(o.w.y, o.s.y)};
                const pair_t ui = {fmaT(-alpha, si.x, o.u.x), fmaT(-alpha, si.y, o.u.y)};
                if (PH)
                    put2(x, i, pair_t{fmaT(alpha, pi.x, fmaT(alpha_prev, o.p.x, o.x.x)),
                                      fmaT(alpha, pi.y, fmaT(alpha_prev, o.p.y, o.x.y))});
                put2(p, i, pi);
                put2(sc, i, si);
                put2(un, i, ui);
                put2(wn, i, pair_t{JAC ? acc0 / a0 : acc0, JAC ? acc1 / a1 : acc1});
                const T r0 = JAC ? a0 * ui.x : ui.x, r1 = JAC ? a1 * ui.y : ui.y;
                g = fma(r0, ui.x, g);
                d = fma(acc0, ui.x, d);
                q = fma(r0, r0, q);
                g = fma(r1, ui.y, g);
                d = fma(acc1, ui.y, d);
                q = fma(r1, r1, q);
            };
            go = dia_rows_pair<SLOTS, true>(
                walk_tiles(pair_tiles_of(n), stopped), n, cg_cols<CM>(A->cols, st),
                [&](int64_t k) { return ld2(val, k); }, [&](int64_t k) { return sld(val, k); },
                [&](int64_t c) { return G3<pair_t>{ld2(uc, c), ld2(wc, c), ld2(sprev, c)}; },
                [&](int64_t c) { return G3<T>{sld(uc, c), sld(wc, c), sld(sprev, c)}; }, u_of,
                [&](int64_t i) {
                    return CgOwn<pair_t>{ld2(uc, i), ld2(wc, i), ld2(sprev, i), ld2(pprev, i),
                                         PH ? ld2((gptr<const T>)x, i) : pair_t{0.0, 0.0}};
                },
                row2, pre, post);
        } else if constexpr (O32) {  // and the +-1 gathers from the adjacent lanes
            go = dia_rows<T, SLOTS, true, true>(
                walk_tiles(tiles_of(n), stopped), n, cg_cols<CM>(A->cols, st),
                [&](auto k) { return ld(val, k); }, gath, u_of, own_of, row, pre, post,
                [&](int64_t k) { return sld(val, k); },
                [&](int64_t c) { return G3<T>{sld(uc, c), sld(wc, c), sld(sprev, c)}; });
        } else {
            go = spmv_rows<T, IT, SLOTS, SLA_CG_ROUND, CM, true>(
                walk_tiles(tiles_of(n), stopped), n, glb(A->rp), cg_cols<CM>(A->cols, st), sm,
                [&](auto k) { return ld(val, k); }, gath, u_of, own_of, row, pre, post);
        }
    }
    if (!go) return;
    double v[3] = {g, d, q};
    const int slot[3] = {PH ? kCgGA : kCgGA1, PH ? kCgDE : kCgDE1, PH ? kCgRR : kCgRR1};
    store_partials<3>(v, part, slot);
}

// x_i = x_{i-1} + alpha_{i-1} p_{i-1} after a stop at an odd iteration i
// (alpha_{i-1} is the parity-0 alpha, p holds p_{i-1}); system blockIdx.y.
template <typename T>
__global__ __launch_bounds__(kBlock) void cg_lag_kernel(const SolveState *st, const T *__restrict__ p,
                                                        T *__restrict__ x, int64_t n) {
    st += blockIdx.y;
    p += (int64_t)blockIdx.y * n;
    x += (int64_t)blockIdx.y * n;
    if (!st->lag) return;
    const T a = (T)st->alpha[0];
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride)
        x[i] = fmaT(a, p[i], x[i]);
}

// ------------------------------------------------------------ split iteration
//
// Patterns with a row plan (rows past the tile walker's stage or slots) run
// the same recurrence as three launches per iteration instead of one: the row
// updates (cg_split_u_kernel), the product w = A u through the products' tile
// kernel and row plan, and the scaled product with the partial sums
// (cg_split_w_kernel).  Scalars, stop tests and partial-sum slots are those of
// cg_iter_kernel; x is brought up to date every iteration (no lag).  Vectors:
// u in r, w^ in q, s^ in s, p in p[0], the raw product in v[0]; t holds A x0.

// r_0 = b - A x_0, u_0 = M^-1 r_0 (A x_0 in t, zeroed without a guess); x = 0
// without an initial guess.
template <typename T, typename IT, bool JAC>
__global__ __launch_bounds__(kBlock) void cg_split_init_kernel(const IterArgs<T, IT> *__restrict__ A) {
    A += blockIdx.y;
    const int64_t n = A->n;
    const TileRange tr = xcd_tiles(tiles_of(n));
    for (int64_t t = tr.first; t < tr.end; t += tr.stride) {
        const int64_t i = t * kTileRows + threadIdx.x;
        if (i >= n) continue;
        const T ri = A->b[i] - A->t[i];
        A->r[i] = JAC ? A->dinv[i] * ri : ri;
        if (!A->use_x0) A->x[i] = T(0);
    }
}

// Iteration i (i = st->iter_p[PH]): the stop tests and scalars of
// cg_iter_kernel, then p_i = u_i + beta p_{i-1}, s^_i = w^_i + beta s^_{i-1},
// u_{i+1} = u_i - alpha s^_i, x_{i+1} = x_i + alpha p_i.
template <typename T, typename IT, bool JAC, int PH>
__global__ __launch_bounds__(kBlock) void cg_split_u_kernel(const IterArgs<T, IT> *__restrict__ A) {
    A += blockIdx.y;
    SolveState *st = A->st;
    __shared__ int seen[kWaves];
    __shared__ double red[4][kWaves];
    const bool stopped = saw_stop(st, seen);
    const int it = st->iter_p[PH];
    const bool first = PH == 0 && it == 0;
    if (!stopped) {
        if (first) {
            const int slot[4] = {kCgGA, kCgDE, kCgRR, kCgBB};
            partial_loads<4>(A->part, slot, red);
        } else {
            const int slot[3] = {PH ? kCgGA1 : kCgGA, PH ? kCgDE1 : kCgDE, PH ? kCgRR1 : kCgRR};
            partial_loads<3>(A->part, slot, red);
        }
    }
    __syncthreads();
    if (any_saw_stop(seen)) return;
    double tot[4];
    if (first) {
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
    if (first && st->zero_diag) {
        finish(st, A->ndone, SLA_ERR_ZERO_DIAG, 0, rr);
        return;
    }
    if (first && bb == 0.0) {
        if (block0()) st->zero_x = A->use_x0 ? 1 : 0;
        finish(st, A->ndone, SLA_OK, 0, 0.0);
        return;
    }
    if (sqrt(rr) <= A->tol * sqrt(bb)) {
        finish(st, A->ndone, SLA_OK, it, rr);
        return;
    }
    if (it >= A->maxit) {
        finish(st, A->ndone, SLA_NOT_CONVERGED, it, rr);
        return;
    }
    const double beta_d = first ? 0.0 : gamma / st->rho[PH ^ 1];
    const double den = first ? delta : delta - beta_d * gamma / st->alpha[PH ^ 1];
    if (!(den > 0.0)) {
        finish(st, A->ndone, SLA_BREAKDOWN, it, rr);
        return;
    }
    const double alpha_d = gamma / den;
    if (block0()) {
        st->rho[PH] = gamma;
        st->alpha[PH] = alpha_d;
        st->iter_p[PH ^ 1] = it + 1;
        st->nfused += 1;
        st->spmv += first ? (A->use_x0 ? 3 : 2) : 1;  // init (and A x0) products
        if (first) st->bb = bb;
    }
    const T beta = (T)beta_d, alpha = (T)alpha_d;
    const int64_t n = A->n;
    const gptr<T> u = glb(A->r), w = glb(A->q), sv = glb(A->s), p = glb(A->p[0]), x = glb(A->x);
    const TileRange tr = xcd_tiles(tiles_of(n));
    for (int64_t t = tr.first; t < tr.end; t += tr.stride) {
        const int64_t i = t * kTileRows + threadIdx.x;
        if (i >= n) continue;
        const T ui = u[i], wi = w[i];
        const T pi = first ? ui : fmaT(beta, p[i], ui);
        const T si = first ? wi : fmaT(beta, sv[i], wi);
        p[i] = pi;
        sv[i] = si;
        u[i] = fmaT(-alpha, si, ui);
        x[i] = fmaT(alpha, pi, x[i]);
    }
}

// After the product w = A u (in v[0]): w^ = w / a_ii (INIT: w * dinv, as
// cg_init_kernel), and the partial sums gamma = r.u, delta = w.u, ||r||^2
// (INIT: r_0 = b - A x0 and also ||b||^2) in the slots cg_iter_kernel uses.
template <typename T, typename IT, bool JAC, int PH, bool INIT>
__global__ __launch_bounds__(kBlock) void cg_split_w_kernel(const IterArgs<T, IT> *__restrict__ A,
                                                            const IT *__restrict__ diagpos) {
    A += blockIdx.y;
    if (!INIT && load_done(A->st)) return;  // set by an earlier launch: uniform
    const int64_t n = A->n;
    const gptr<const T> wraw = glb((const T *)A->v[0]);
    const gptr<const T> u = glb((const T *)A->r);
    const gptr<T> w = glb(A->q);
    double g = 0.0, d = 0.0, q = 0.0, bb = 0.0;
    const TileRange tr = xcd_tiles(tiles_of(n));
    for (int64_t t = tr.first; t < tr.end; t += tr.stride) {
        const int64_t i = t * kTileRows + threadIdx.x;
        if (i >= n) continue;
        const T acc = wraw[i], ui = u[i];
        if (INIT) {
            const T bi = A->b[i];
            const T ri = bi - A->t[i];
            w[i] = JAC ? acc * A->dinv[i] : acc;
            g = fma((double)ri, (double)ui, g);
            d = fma((double)acc, (double)ui, d);
            q = fma((double)ri, (double)ri, q);
            bb = fma((double)bi, (double)bi, bb);
        } else {
            const T aii = JAC ? A->val[diagpos[i]] : T(1);
            w[i] = JAC ? acc / aii : acc;
            const T ri = JAC ? aii * ui : ui;
            g = fma((double)ri, (double)ui, g);
            d = fma((double)acc, (double)ui, d);
            q = fma((double)ri, (double)ri, q);
        }
    }
    if (INIT) {
        double v[4] = {g, d, q, bb};
        const int slot[4] = {kCgGA, kCgDE, kCgRR, kCgBB};
        store_partials<4>(v, A->part, slot);
    } else {
        double v[3] = {g, d, q};
        const int slot[3] = {PH ? kCgGA : kCgGA1, PH ? kCgDE : kCgDE1, PH ? kCgRR : kCgRR1};
        store_partials<3>(v, A->part, slot);
    }
}

// ------------------------------------------------------------------ launchers

// Planes per workgroup below which the z-walk is not used.  A segment reads
// the plane below its first one and the plane above its last one, which its
// neighbouring segments load at the other end of their walks, by then out
// of L2: with short segments these reloads cost more than the ring saves
// (100^3, 4 planes per segment: 94.7 MB read per launch instead of the
// 80.1 MB of the tiles in slabs, 25.2 instead of 24.5 us).
constexpr int64_t kZwMinPlanes = 16;
// Working sets beyond this stay out of the 256 MB Infinity Cache.
constexpr int64_t kInfinityCacheBytes = (int64_t)256 << 20;

int cg_zwalk_plan(ColArgs &it, int64_t n, int64_t value_bytes) {
    it.zw_tw = it.zw_ncol = it.zw_nseg = it.zw_nz = 0;
    if (it.mode != kColDiaMajor || it.nd != 7) return 0;
    const int64_t D = it.off[6];
    if (!(it.off[2] == -1 && it.off[4] == 1 && it.off[0] == -D && it.off[1] == -it.off[5] &&
          it.off[5] > 1 && D > it.off[5] && n % D == 0))
        return 0;
    const int64_t nz = n / D;
    const int64_t grid = grid_for_tiles(tiles_of(n));
    const int64_t ncol = (D + kTileRows - 1) / kTileRows;  // columns of at most 256 rows
    const int64_t tw = (D + ncol - 1) / ncol;                // as even as they go
    int64_t nseg = grid / ncol;                              // segments per column
    if (nseg < 1 || nz / nseg < kZwMinPlanes) return 0;
    it.zw_tw = (int32_t)tw;
    it.zw_ncol = (int32_t)ncol;
    it.zw_nseg = (int32_t)nseg;
    it.zw_nz = (int32_t)nz;
    // the iteration touches 4 values (symmetric: main and upper diagonals)
    // and 9 vectors of each row on average
    return n * 13 * value_bytes > kInfinityCacheBytes ? 2 : 1;
}

template <typename T, typename IT>
hipError_t launch_cg_init(int slots, int cm, int zw, bool jac, const IterArgs<T, IT> *a,
                          int64_t n, int nsys, hipStream_t s) {
    const dim3 grid(iter_grid(cm, zw, n), nsys);  // the iterations' grid (partial sums)
    if (jac) {
        SLA_DISPATCH_FORM(cm, slots, cg_init_kernel<T, IT, true, kS, kC>
                                                 <<<grid, kBlock, 0, s>>>(a));
    } else {
        SLA_DISPATCH_FORM(cm, slots, cg_init_kernel<T, IT, false, kS, kC>
                                                 <<<grid, kBlock, 0, s>>>(a));
    }
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_cg_iter(int slots, int cm, bool jac, int zw, int tile,
                          const IterArgs<T, IT> *a, int64_t n, int nsys, int ph, hipStream_t s,
                          const hipEvent_t *ev) {
    const dim3 grid(iter_grid(cm, zw, n), nsys);
    const bool o32 = tile != kDiaTileGeneral && cm == kColDiaMajor && zw == 0;
    // row pairs: fp64 only (dia_tile never asks them for other types)
    const bool pair = sizeof(T) == 8 && o32 && tile == kDiaTilePair;
#define SLA_CG_O32(J, P, S)                                                                     \
    do {                                                                                        \
        if constexpr (sizeof(T) == 8) {                                                         \
            if (pair) {                                                                         \
                launch_maybe_timed(cg_iter_kernel<T, IT, J, S, P, kColDiaMajor, 0, true, true>, \
                                   grid, dim3(kBlock), 0, s, ev, a);                            \
                break;                                                                          \
            }                                                                                   \
        }                                                                                       \
        launch_maybe_timed(cg_iter_kernel<T, IT, J, S, P, kColDiaMajor, 0, true>, grid,        \
                           dim3(kBlock), 0, s, ev, a);                                          \
    } while (0)
#define SLA_CG_ITER(J, P)                                                                      \
    if (zw == 2)                                                                               \
        launch_maybe_timed(cg_iter_kernel<T, IT, J, 7, P, kColDiaMajor, 2>, grid,              \
                           dim3(kBlock), 0, s, ev, a);                                         \
    else if (zw == 1)                                                                          \
        launch_maybe_timed(cg_iter_kernel<T, IT, J, 7, P, kColDiaMajor, 1>, grid,              \
                           dim3(kBlock), 0, s, ev, a);                                         \
    else if (o32 && slots == 3)                                                                \
        SLA_CG_O32(J, P, 3);                                                                   \
    else if (o32 && slots == 5)                                                                \
        SLA_CG_O32(J, P, 5);                                                                   \
    else if (o32)                                                                              \
        SLA_CG_O32(J, P, 7);                                                                   \
    else                                                                                       \
        SLA_DISPATCH_FORM(cm, slots, launch_maybe_timed(cg_iter_kernel<T, IT, J, kS, P, kC>,   \
                                                        grid, dim3(kBlock), 0, s, ev, a))
    if (jac) {
        if (ph) {
            SLA_CG_ITER(true, 1);
        } else {
            SLA_CG_ITER(true, 0);
        }
    } else {
        if (ph) {
            SLA_CG_ITER(false, 1);
        } else {
            SLA_CG_ITER(false, 0);
        }
    }
#undef SLA_CG_ITER
#undef SLA_CG_O32
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_cg_split_init(bool jac, const IterArgs<T, IT> *a, int64_t n, int nsys,
                                hipStream_t s) {
    const dim3 grid(grid_for_tiles(tiles_of(n)), nsys);
    if (jac)
        cg_split_init_kernel<T, IT, true><<<grid, kBlock, 0, s>>>(a);
    else
        cg_split_init_kernel<T, IT, false><<<grid, kBlock, 0, s>>>(a);
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_cg_split_u(bool jac, const IterArgs<T, IT> *a, int64_t n, int nsys, int ph,
                             hipStream_t s) {
    const dim3 grid(grid_for_tiles(tiles_of(n)), nsys);
    if (jac) {
        if (ph)
            cg_split_u_kernel<T, IT, true, 1><<<grid, kBlock, 0, s>>>(a);
        else
            cg_split_u_kernel<T, IT, true, 0><<<grid, kBlock, 0, s>>>(a);
    } else {
        if (ph)
            cg_split_u_kernel<T, IT, false, 1><<<grid, kBlock, 0, s>>>(a);
        else
            cg_split_u_kernel<T, IT, false, 0><<<grid, kBlock, 0, s>>>(a);
    }
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_cg_split_w(bool jac, bool init, const IterArgs<T, IT> *a, const IT *diagpos,
                             int64_t n, int nsys, int ph, hipStream_t s) {
    const dim3 grid(grid_for_tiles(tiles_of(n)), nsys);
#define SLA_SPLIT_W(J)                                                                   \
    if (init)                                                                            \
        cg_split_w_kernel<T, IT, J, 0, true><<<grid, kBlock, 0, s>>>(a, diagpos);        \
    else if (ph)                                                                         \
        cg_split_w_kernel<T, IT, J, 1, false><<<grid, kBlock, 0, s>>>(a, diagpos);       \
    else                                                                                 \
        cg_split_w_kernel<T, IT, J, 0, false><<<grid, kBlock, 0, s>>>(a, diagpos)
    if (jac) {
        SLA_SPLIT_W(true);
    } else {
        SLA_SPLIT_W(false);
    }
#undef SLA_SPLIT_W
    return hipGetLastError();
}

template <typename T>
hipError_t launch_cg_lag(const SolveState *st, const T *p, T *x, int64_t n, int nsys,
                         hipStream_t s) {
    int64_t blocks = (n + kBlock - 1) / kBlock;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    cg_lag_kernel<T><<<dim3((unsigned)blocks, nsys), kBlock, 0, s>>>(st, p, x, n);
    return hipGetLastError();
}
template hipError_t launch_cg_lag<float>(const SolveState *, const float *, float *, int64_t, int,
                                         hipStream_t);
template hipError_t launch_cg_lag<double>(const SolveState *, const double *, double *, int64_t,
                                          int, hipStream_t);

#define SLA_INST(T, IT)                                                                         \
    template hipError_t launch_cg_init<T, IT>(int, int, int, bool, const IterArgs<T, IT> *,  \
                                              int64_t, int, hipStream_t);                       \
    template hipError_t launch_cg_iter<T, IT>(int, int, bool, int, int,                     \
                                              const IterArgs<T, IT> *, int64_t, int, int,       \
                                              hipStream_t, const hipEvent_t *);                 \
    template hipError_t launch_cg_split_init<T, IT>(bool, const IterArgs<T, IT> *, int64_t, int, \
                                                    hipStream_t);                              \
    template hipError_t launch_cg_split_u<T, IT>(bool, const IterArgs<T, IT> *, int64_t, int,    \
                                                 int, hipStream_t);                            \
    template hipError_t launch_cg_split_w<T, IT>(bool, bool, const IterArgs<T, IT> *, const IT *, \
                                                 int64_t, int, int, hipStream_t);

SLA_INST(float, int32_t)
SLA_INST(float, int64_t)
SLA_INST(double, int32_t)
SLA_INST(double, int64_t)

}  // namespace sla
