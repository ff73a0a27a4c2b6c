// BiCGStab for nonsymmetric systems (torch-sla explainer, Methodology
// section 1 lists BiCGStab among the iterative solvers; steps of van der
// Vorst, SIAM J. Sci. Stat. Comput. 13, 1992), unpreconditioned, grid path.
//
// Two kernels per iteration j (0-based), each one product and one set of
// partial sums:
//   bicg_xpv (iteration j): from the partials of iteration j-1,
//            omega = t.s / t.t; half-step exit (||s|| <= tol ||b||:
//            x += alpha p, stop in the next kernel); else x_j = x + alpha p
//            + omega s, r_j = s - omega t (evaluated while gathering as
//            well), rho_j = rhat.r_j = rhat.s - omega rhat.t, beta_j =
//            (rho_j / rho_{j-1}) (alpha_{j-1} / omega), p_j = r_j + beta_j
//            (p - omega v) evaluated while gathering, v_j = A p_j; partials
//            rhat.v_j and ||r_j||^2.  At j = 0, r_0 is read as stored and
//            rho_0 = ||r_0||^2 (rhat = r_0) comes from the init partials.
//   bicg_st  (iteration j): stop tests on the exact ||r_j|| (converged, maxit,
//            rho_j = 0 or NaN); alpha_j = rho_j / rhat.v_j; s = r_j - alpha v_j
//            evaluated while gathering, t = A s; partials t.s, t.t, s.s,
//            rhat.s, rhat.t.
// The textbook's third reduction (rhat.r_j after the r update) comes from
// the st partials through the identity rhat.(s - omega t) = rhat.s -
// omega rhat.t, so the r and x updates fold into the next iteration's first
// kernel; the iterates are those of the textbook in exact arithmetic, and
// every stop decision uses the same dots as the textbook (||r_j||^2 summed
// from r_j itself, one kernel later).  Each kernel stores per-block partial
// sums; every block of the next kernel adds them in the same order, so the
// scalars are identical everywhere and no kernel needs a grid-wide fence.
// p and v are double-buffered by iteration parity (the product kernels read
// the old vectors at neighbouring rows while they write the new ones); r is
// written only by bicg_xpv at j >= 1, whose gathers read s and t.  A launch
// advances a group of systems, one per row of the grid's y dimension, each
// through its own argument block (vectors, state and partial sums of its
// own); a system that has stopped ends each later launch at its first
// barrier.
#include "spmv_tile.h"

namespace sla {

template <typename T>
__device__ __forceinline__ T fmaB(T a, T b, T c) {
    return fma(a, b, c);
}

// A Krylov denominator that vanished: zero, or NaN (a NaN or an infinity in
// b or in the values turns the dots into NaN within an iteration or two; the
// iteration can divide by neither).
__device__ __forceinline__ bool vanished(double d) { return !(fabs(d) > 0.0); }

// r = rhat = b - A x0 (or b with x = 0); partials ||r||^2 (= rhat.r) and b.b.
template <typename T, typename IT>
__global__ __launch_bounds__(kBlock) void bicg_init_kernel(const IterArgs<T, IT> *__restrict__ A) {
    A += blockIdx.y;  // system blockIdx.y of the launch
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
            rr = fma((double)ri, (double)ri, rr);
            bb = fma((double)bi, (double)bi, bb);
        }
    }
    double v[2] = {rr, bb};
    const int slot[2] = {kBiRR0, kBiBB};
    store_partials<2>(v, A->part, slot);
}

// A row's own inputs of bicg_xpv (the gathers take s, t, p and v as a G4).
template <typename T>
struct XpvOwn {
    T s, t, p, v, x, rh;
};

#ifndef SLA_BICG_WAVES
#define SLA_BICG_WAVES 5
#endif
// O32 (both kernels): the fast diagonal-major tiles (dia_tile): 32-bit byte
// offsets (elem) and the +-1 gathers from the adjacent lanes (dia_rows ADJ);
// PAIR: the same with two rows per lane (fp64, dia_rows_pair).
template <typename T, typename IT, int SLOTS, int CM, bool O32 = false, bool PAIR = false>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(CM == kColDiaMajor ? 3 : SLA_BICG_WAVES)))
void bicg_xpv_kernel(const IterArgs<T, IT> *__restrict__ A) {
    A += blockIdx.y;  // system blockIdx.y of the launch
    SolveState *st = A->st;
    __shared__ int seen[kWaves];
    const bool stopped = saw_stop(st, seen);
    const int it = st->iter_a;
    const bool first = (it == 0);
    const int64_t n = A->n;
    const gptr<const T> val = glb(A->val);
    const gptr<const T> rh = glb((const T *)A->rh);
    // at j = 0 every gathered vector is r_0: with omega = beta = 0 the
    // expressions below give r_0 and p_0 = r_0 exactly
    const gptr<const T> sv = first ? glb((const T *)A->r) : glb((const T *)A->s);
    const gptr<const T> tv = first ? sv : glb((const T *)A->t);
    const gptr<const T> pold = first ? sv : glb((const T *)A->p[it & 1]);
    const gptr<const T> vold = first ? sv : glb((const T *)A->v[it & 1]);
    const gptr<T> pnew = glb(A->p[(it + 1) & 1]);
    const gptr<T> vnew = glb(A->v[(it + 1) & 1]);
    const gptr<T> x = glb(A->x);
    const gptr<T> r = glb(A->r);
    __shared__ RowLds<T, IT> sm;
    __shared__ double red[5][kWaves];
    auto pre = [&]() {
        if (stopped) return;
        if (first) {
            const int slot[2] = {kBiRR0, kBiBB};
            partial_loads<2>(A->part, slot, red);
        } else {
            const int slot[5] = {kBiTS, kBiTT, kBiSS, kBiRS, kBiRT};
            partial_loads<5>(A->part, slot, red);
        }
    };
    T alpha = T(0), omega = T(0), beta = T(0);
    auto post = [&]() -> bool {
        if (any_saw_stop(seen)) return false;
        if (first) {
            double tot[2];
            totals<2>(red, tot);
            const double rr = tot[0], bb = tot[1];
            if (bb == 0.0) {
                if (block0()) st->zero_x = A->use_x0 ? 1 : 0;
                finish(st, A->ndone, SLA_OK, 0, 0.0);
                return false;
            }
            if (block0()) {
                st->rho[0] = rr;  // rhat = r_0
                st->bb = bb;
                st->iter_b = 0;
                st->spmv += A->use_x0 ? 1 : 0;  // the A x0 product
                st->nfused += 1;
            }
            return true;
        }
        double tot[5];
        totals<5>(red, tot);
        const double ts = tot[0], tt = tot[1], ss = tot[2], rs = tot[3], rt = tot[4];
        const int pv = (it + 1) & 1;  // parity slot of iteration j - 1
        alpha = (T)st->alpha[pv];
        if (sqrt(ss) <= A->tol * sqrt(st->bb)) {
            // half step: x_j = x + alpha p; the next kernel stops (a block
            // still to start must not see `done` before its x update)
            const TileRange tr = xcd_tiles(tiles_of(n));
            for (int64_t t = tr.first; t < tr.end; t += tr.stride) {
                const int64_t i = t * kTileRows + threadIdx.x;
                if (i < n) x[i] = fmaB(alpha, pold[i], x[i]);
            }
            if (block0()) {
                st->half_ss = ss;
                st->half_exit = 1;
                st->iter_b = it;
            }
            return false;
        }
        if (vanished(tt) || vanished(ts)) {
            if (block0()) st->spmv += 1;  // the t product of iteration j - 1
            finish(st, A->ndone, SLA_BREAKDOWN, it - 1, 0.0);
            return false;
        }
        const double omega_d = ts / tt;
        const double rho = rs - omega_d * rt;
        omega = (T)omega_d;
        beta = (T)((rho / st->rho[pv]) * (st->alpha[pv] / omega_d));
        if (block0()) {
            st->rho[it & 1] = rho;
            st->iter_b = it;
            st->spmv += 1;  // the t product of iteration j - 1
            st->nfused += 1;
        }
        return true;
    };
    // r_j and p_j at one index from s, t, the previous p and v
    auto rj = [&](T sa, T ta) -> T { return fmaB(-omega, ta, sa); };
    auto pj = [&](const G4<T> &g) -> T {
        return fmaB(beta, fmaB(-omega, g.d, g.c), rj(g.a, g.b));
    };
    double rv_acc = 0.0, rr_acc = 0.0;
    auto ld = [&](gptr<const T> v, int64_t i) -> T { return *elem<O32>(v, i); };
    if constexpr (PAIR) {
        static_assert(O32 && sizeof(T) == 8, "row pairs: fast fp64 tiles");
        auto ld2 = [&](gptr<const T> v, int64_t i) -> pair_t {
            return *(const __attribute__((address_space(1))) pair_t *)elem<O32>(v, i);
        };
        auto put2 = [&](gptr<T> v, int64_t i, pair_t a) {
            *(__attribute__((address_space(1))) pair_t *)elem<O32>(v, i) = a;
        };
        const bool go = dia_rows_pair<SLOTS, false>(
            walk_tiles(pair_tiles_of(n), stopped), n, col_src<CM>(A->cols),
            [&](int64_t k) { return ld2(val, k); }, nullptr,
            [&](int64_t c) {
                return G4<pair_t>{ld2(sv, c), ld2(tv, c), ld2(pold, c), ld2(vold, c)};
            },
            [&](int64_t c) { return G4<T>{sld(sv, c), sld(tv, c), sld(pold, c), sld(vold, c)}; },
            pj,
            [&](int64_t i) {
                return XpvOwn<pair_t>{ld2(sv, i), ld2(tv, i), ld2(pold, i), ld2(vold, i),
                                      first ? pair_t{0.0, 0.0} : ld2((gptr<const T>)x, i),
                                      ld2(rh, i)};
            },
            [&](int64_t i, T acc0, T acc1, const XpvOwn<pair_t> &o, T, T) {
                const pair_t ri = {rj(o.s.x, o.t.x), rj(o.s.y, o.t.y)};
                if (!first) {
                    put2(x, i, pair_t{fmaB(omega, o.s.x, fmaB(alpha, o.p.x, o.x.x)),
                                      fmaB(omega, o.s.y, fmaB(alpha, o.p.y, o.x.y))});
                    put2(r, i, ri);
                }
                put2(pnew, i, pair_t{pj(G4<T>{o.s.x, o.t.x, o.p.x, o.v.x}),
                                     pj(G4<T>{o.s.y, o.t.y, o.p.y, o.v.y})});
                put2(vnew, i, pair_t{acc0, acc1});
                rv_acc = fma(o.rh.x, acc0, rv_acc);
                rr_acc = fma(ri.x, ri.x, rr_acc);
                rv_acc = fma(o.rh.y, acc1, rv_acc);
                rr_acc = fma(ri.y, ri.y, rr_acc);
            },
            pre, post);
        if (!go) return;
        double v[2] = {rv_acc, rr_acc};
        const int slot[2] = {kBiRV, kBiRR};
        store_partials<2>(v, A->part, slot);
        return;
    }
    auto rows = [&](auto vf, auto gf, auto of, auto rf) {
        if constexpr (O32)  // and the +-1 gathers from the adjacent lanes
            return dia_rows<T, SLOTS, false, true>(
                walk_tiles(tiles_of(n), stopped), n, col_src<CM>(A->cols), vf, gf, pj, of, rf,
                pre, post, nullptr, [&](int64_t c) {
                    return G4<T>{sld(sv, c), sld(tv, c), sld(pold, c), sld(vold, c)};
                });
        else
            return spmv_rows<T, IT, SLOTS, 4>(walk_tiles(tiles_of(n), stopped), n, glb(A->rp),
                                              col_src<CM>(A->cols), sm, vf, gf, pj, of, rf, pre,
                                              post);
    };
    const bool go = rows(
        [&](auto k) { return ld(val, k); },
        [&](int32_t c) { return G4<T>{ld(sv, c), ld(tv, c), ld(pold, c), ld(vold, c)}; },
        [&](int64_t i) {
            return XpvOwn<T>{ld(sv, i), ld(tv, i), ld(pold, i), ld(vold, i),
                             first ? T(0) : ld((gptr<const T>)x, i), ld(rh, i)};
        },
        [&](int64_t i, T acc, const XpvOwn<T> &o, T) {
            const T ri = rj(o.s, o.t);
            if (!first) {
                *elem<O32>(x, i) = fmaB(omega, o.s, fmaB(alpha, o.p, o.x));
                *elem<O32>(r, i) = ri;
            }
            *elem<O32>(pnew, i) = pj(G4<T>{o.s, o.t, o.p, o.v});
            *elem<O32>(vnew, i) = acc;
            rv_acc = fma((double)o.rh, (double)acc, rv_acc);
            rr_acc = fma((double)ri, (double)ri, rr_acc);
        });
    if (!go) return;
    double v[2] = {rv_acc, rr_acc};
    const int slot[2] = {kBiRV, kBiRR};
    store_partials<2>(v, A->part, slot);
}

template <typename T>
struct StOwn {
    T r, v, rh;
};

// Iteration j (j = iter_b): a pending half-step exit stops here; stop tests
// on ||r_j|| (converged, then maxit) and rho_j = 0 (breakdown);
// alpha_j = rho_j / rhat.v_j (rhat.v_j = 0: breakdown); s = r - alpha v
// evaluated while gathering, t = A s; partials t.s, t.t, s.s, rhat.s, rhat.t.
template <typename T, typename IT, int SLOTS, int CM, bool O32 = false, bool PAIR = false>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(CM == kColDiaMajor ? 3 : SLA_BICG_WAVES)))
void bicg_st_kernel(const IterArgs<T, IT> *__restrict__ A) {
    A += blockIdx.y;  // system blockIdx.y of the launch
    SolveState *st = A->st;
    __shared__ int seen[kWaves];
    const bool stopped = saw_stop(st, seen);
    const int it = st->iter_b;
    const int64_t n = A->n;
    const gptr<const T> val = glb(A->val);
    const gptr<const T> r = glb((const T *)A->r);
    const gptr<const T> rh = glb((const T *)A->rh);
    const gptr<const T> v = glb((const T *)A->v[(it + 1) & 1]);
    const gptr<T> s = glb(A->s);
    const gptr<T> tv = glb(A->t);
    __shared__ RowLds<T, IT> sm;
    __shared__ double red[2][kWaves];
    auto pre = [&]() {
        if (stopped) return;
        const int slot[2] = {kBiRV, kBiRR};
        partial_loads<2>(A->part, slot, red);
    };
    T alpha = T(0);
    auto post = [&]() -> bool {
        if (any_saw_stop(seen)) return false;
        if (st->half_exit) {
            finish(st, A->ndone, SLA_OK, it, st->half_ss);
            return false;
        }
        double tot[2];
        totals<2>(red, tot);
        const double rv = tot[0], rr = tot[1];
        if (sqrt(rr) <= A->tol * sqrt(st->bb)) {
            finish(st, A->ndone, SLA_OK, it, rr);
            return false;
        }
        if (it >= A->maxit) {
            finish(st, A->ndone, SLA_NOT_CONVERGED, it, rr);
            return false;
        }
        const double rho = st->rho[it & 1];
        if (vanished(rho)) {
            finish(st, A->ndone, SLA_BREAKDOWN, it, rr);
            return false;
        }
        if (block0()) st->spmv += 1;  // v_j = A p_j
        if (vanished(rv)) {
            finish(st, A->ndone, SLA_BREAKDOWN, it, rr);
            return false;
        }
        const double alpha_d = rho / rv;
        alpha = (T)alpha_d;
        if (block0()) {
            st->alpha[it & 1] = alpha_d;
            st->iter_a = it + 1;
            st->nfused += 1;
        }
        return true;
    };
    auto sk = [&](const G2<T> &g) -> T { return fmaB(-alpha, g.b, g.a); };
    double ts = 0.0, tt = 0.0, ss = 0.0, rs = 0.0, rt = 0.0;
    auto ld = [&](gptr<const T> w, int64_t i) -> T { return *elem<O32>(w, i); };
    if constexpr (PAIR) {
        static_assert(O32 && sizeof(T) == 8, "row pairs: fast fp64 tiles");
        auto ld2 = [&](gptr<const T> w, int64_t i) -> pair_t {
            return *(const __attribute__((address_space(1))) pair_t *)elem<O32>(w, i);
        };
        auto put2 = [&](gptr<T> w, int64_t i, pair_t a) {
            *(__attribute__((address_space(1))) pair_t *)elem<O32>(w, i) = a;
        };
        const bool go = dia_rows_pair<SLOTS, false>(
            walk_tiles(pair_tiles_of(n), stopped), n, col_src<CM>(A->cols),
            [&](int64_t k) { return ld2(val, k); }, nullptr,
            [&](int64_t c) { return G2<pair_t>{ld2(r, c), ld2(v, c)}; },
            [&](int64_t c) { return G2<T>{sld(r, c), sld(v, c)}; }, sk,
            [&](int64_t i) { return StOwn<pair_t>{ld2(r, i), ld2(v, i), ld2(rh, i)}; },
            [&](int64_t i, T acc0, T acc1, const StOwn<pair_t> &o, T, T) {
                const pair_t si = {sk(G2<T>{o.r.x, o.v.x}), sk(G2<T>{o.r.y, o.v.y})};
                put2(s, i, si);
                put2(tv, i, pair_t{acc0, acc1});
                const T sh[2] = {si.x, si.y}, ah[2] = {acc0, acc1}, rhh[2] = {o.rh.x, o.rh.y};
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    ts = fma(ah[h], sh[h], ts);
                    tt = fma(ah[h], ah[h], tt);
                    ss = fma(sh[h], sh[h], ss);
                    rs = fma(rhh[h], sh[h], rs);
                    rt = fma(rhh[h], ah[h], rt);
                }
            },
            pre, post);
        if (!go) return;
        double red5[5] = {ts, tt, ss, rs, rt};
        const int slot[5] = {kBiTS, kBiTT, kBiSS, kBiRS, kBiRT};
        store_partials<5>(red5, A->part, slot);
        return;
    }
    auto rows = [&](auto vf, auto gf, auto of, auto rf) {
        if constexpr (O32)  // and the +-1 gathers from the adjacent lanes
            return dia_rows<T, SLOTS, false, true>(
                walk_tiles(tiles_of(n), stopped), n, col_src<CM>(A->cols), vf, gf, sk, of, rf,
                pre, post, nullptr, [&](int64_t c) { return G2<T>{sld(r, c), sld(v, c)}; });
        else
            return spmv_rows<T, IT, SLOTS, SLOTS>(walk_tiles(tiles_of(n), stopped), n,
                                                  glb(A->rp), col_src<CM>(A->cols), sm, vf, gf,
                                                  sk, of, rf, pre, post);
    };
    const bool go = rows(
        [&](auto k) { return ld(val, k); },
        [&](int32_t c) { return G2<T>{ld(r, c), ld(v, c)}; },
        [&](int64_t i) { return StOwn<T>{ld(r, i), ld(v, i), ld(rh, i)}; },
        [&](int64_t i, T acc, const StOwn<T> &o, T) {
            const T si = sk(G2<T>{o.r, o.v});
            *elem<O32>(s, i) = si;
            *elem<O32>(tv, i) = acc;
            ts = fma((double)acc, (double)si, ts);
            tt = fma((double)acc, (double)acc, tt);
            ss = fma((double)si, (double)si, ss);
            rs = fma((double)o.rh, (double)si, rs);
            rt = fma((double)o.rh, (double)acc, rt);
        });
    if (!go) return;
    double red5[5] = {ts, tt, ss, rs, rt};
    const int slot[5] = {kBiTS, kBiTT, kBiSS, kBiRS, kBiRT};
    store_partials<5>(red5, A->part, slot);
}

// ------------------------------------------------------------ split iteration
//
// Operators with a row plan (rows past the tile walker's stage or slots):
// each kernel above becomes three launches, its row updates, the product
// through the products' tile kernel and row plan, and its partial sums.  The
// stop tests, scalars and partial-sum slots are those of the fused kernels.
// The product of iteration j's first half is p_j -> v_j (buffers p and v of
// parity (j + 1) & 1, which the host picks: split chunks start at even j),
// of its second half s -> t.

// bicg_xpv's tests and scalars, then x_j, r_j and p_j per row.
template <typename T, typename IT>
__global__ __launch_bounds__(kBlock) void bicg_split_xpv_u_kernel(const IterArgs<T, IT> *__restrict__ A) {
    A += blockIdx.y;  // system blockIdx.y of the launch
    SolveState *st = A->st;
    __shared__ int seen[kWaves];
    __shared__ double red[5][kWaves];
    const bool stopped = saw_stop(st, seen);
    const int it = st->iter_a;
    const bool first = (it == 0);
    const int64_t n = A->n;
    const gptr<const T> sv = first ? glb((const T *)A->r) : glb((const T *)A->s);
    const gptr<const T> tv = first ? sv : glb((const T *)A->t);
    const gptr<const T> pold = first ? sv : glb((const T *)A->p[it & 1]);
    const gptr<const T> vold = first ? sv : glb((const T *)A->v[it & 1]);
    const gptr<T> pnew = glb(A->p[(it + 1) & 1]);
    const gptr<T> x = glb(A->x);
    const gptr<T> r = glb(A->r);
    if (!stopped) {
        if (first) {
            const int slot[2] = {kBiRR0, kBiBB};
            partial_loads<2>(A->part, slot, red);
        } else {
            const int slot[5] = {kBiTS, kBiTT, kBiSS, kBiRS, kBiRT};
            partial_loads<5>(A->part, slot, red);
        }
    }
    __syncthreads();
    if (any_saw_stop(seen)) return;
    T alpha = T(0), omega = T(0), beta = T(0);
    const TileRange tr = xcd_tiles(tiles_of(n));
    if (first) {
        double tot[2];
        totals<2>(red, tot);
        const double rr = tot[0], bb = tot[1];
        if (bb == 0.0) {
            if (block0()) st->zero_x = A->use_x0 ? 1 : 0;
            finish(st, A->ndone, SLA_OK, 0, 0.0);
            return;
        }
        if (block0()) {
            st->rho[0] = rr;  // rhat = r_0
            st->bb = bb;
            st->iter_b = 0;
            st->spmv += A->use_x0 ? 1 : 0;  // the A x0 product
            st->nfused += 1;
        }
    } else {
        double tot[5];
        totals<5>(red, tot);
        const double ts = tot[0], tt = tot[1], ss = tot[2], rs = tot[3], rt = tot[4];
        const int pv = (it + 1) & 1;  // parity slot of iteration j - 1
        alpha = (T)st->alpha[pv];
        if (sqrt(ss) <= A->tol * sqrt(st->bb)) {
            // half step: x_j = x + alpha p; the next launches stop
            for (int64_t t = tr.first; t < tr.end; t += tr.stride) {
                const int64_t i = t * kTileRows + threadIdx.x;
                if (i < n) x[i] = fmaB(alpha, pold[i], x[i]);
            }
            if (block0()) {
                st->half_ss = ss;
                st->half_exit = 1;
                st->iter_b = it;
            }
            return;
        }
        if (vanished(tt) || vanished(ts)) {
            if (block0()) st->spmv += 1;  // the t product of iteration j - 1
            finish(st, A->ndone, SLA_BREAKDOWN, it - 1, 0.0);
            return;
        }
        const double omega_d = ts / tt;
        const double rho = rs - omega_d * rt;
        omega = (T)omega_d;
        beta = (T)((rho / st->rho[pv]) * (st->alpha[pv] / omega_d));
        if (block0()) {
            st->rho[it & 1] = rho;
            st->iter_b = it;
            st->spmv += 1;  // the t product of iteration j - 1
            st->nfused += 1;
        }
    }
    for (int64_t t = tr.first; t < tr.end; t += tr.stride) {
        const int64_t i = t * kTileRows + threadIdx.x;
        if (i >= n) continue;
        const T si = sv[i], ti = tv[i], pi = pold[i], vi = vold[i];
        const T ri = fmaB(-omega, ti, si);
        if (!first) {
            x[i] = fmaB(omega, si, fmaB(alpha, pi, x[i]));
            r[i] = ri;
        }
        pnew[i] = fmaB(beta, fmaB(-omega, vi, pi), ri);
    }
}

// After v_j = A p_j: partials rhat.v_j and ||r_j||^2.
template <typename T, typename IT>
__global__ __launch_bounds__(kBlock) void bicg_split_xpv_w_kernel(const IterArgs<T, IT> *__restrict__ A) {
    A += blockIdx.y;  // system blockIdx.y of the launch
    SolveState *st = A->st;
    if (load_done(st) || st->half_exit) return;  // set by an earlier launch: uniform
    const int it = st->iter_a;
    const int64_t n = A->n;
    const gptr<const T> vnew = glb((const T *)A->v[(it + 1) & 1]);
    const gptr<const T> r = glb((const T *)A->r);
    const gptr<const T> rh = glb((const T *)A->rh);
    double rv = 0.0, rr = 0.0;
    const TileRange tr = xcd_tiles(tiles_of(n));
    for (int64_t t = tr.first; t < tr.end; t += tr.stride) {
        const int64_t i = t * kTileRows + threadIdx.x;
        if (i >= n) continue;
        const T ri = r[i];
        rv = fma((double)rh[i], (double)vnew[i], rv);
        rr = fma((double)ri, (double)ri, rr);
    }
    double v[2] = {rv, rr};
    const int slot[2] = {kBiRV, kBiRR};
    store_partials<2>(v, A->part, slot);
}

// bicg_st's tests and alpha_j, then s = r_j - alpha_j v_j per row.
template <typename T, typename IT>
__global__ __launch_bounds__(kBlock) void bicg_split_st_u_kernel(const IterArgs<T, IT> *__restrict__ A) {
    A += blockIdx.y;  // system blockIdx.y of the launch
    SolveState *st = A->st;
    __shared__ int seen[kWaves];
    __shared__ double red[2][kWaves];
    const bool stopped = saw_stop(st, seen);
    const int it = st->iter_b;
    const int64_t n = A->n;
    if (!stopped) {
        const int slot[2] = {kBiRV, kBiRR};
        partial_loads<2>(A->part, slot, red);
    }
    __syncthreads();
    if (any_saw_stop(seen)) return;
    if (st->half_exit) {
        finish(st, A->ndone, SLA_OK, it, st->half_ss);
        return;
    }
    double tot[2];
    totals<2>(red, tot);
    const double rv = tot[0], rr = tot[1];
    if (sqrt(rr) <= A->tol * sqrt(st->bb)) {
        finish(st, A->ndone, SLA_OK, it, rr);
        return;
    }
    if (it >= A->maxit) {
        finish(st, A->ndone, SLA_NOT_CONVERGED, it, rr);
        return;
    }
    const double rho = st->rho[it & 1];
    if (vanished(rho)) {
        finish(st, A->ndone, SLA_BREAKDOWN, it, rr);
        return;
    }
    if (block0()) st->spmv += 1;  // v_j = A p_j
    if (vanished(rv)) {
        finish(st, A->ndone, SLA_BREAKDOWN, it, rr);
        return;
    }
    const double alpha_d = rho / rv;
    const T alpha = (T)alpha_d;
    if (block0()) {
        st->alpha[it & 1] = alpha_d;
        st->iter_a = it + 1;
        st->nfused += 1;
    }
    const gptr<const T> r = glb((const T *)A->r);
    const gptr<const T> v = glb((const T *)A->v[(it + 1) & 1]);
    const gptr<T> s = glb(A->s);
    const TileRange tr = xcd_tiles(tiles_of(n));
    for (int64_t t = tr.first; t < tr.end; t += tr.stride) {
        const int64_t i = t * kTileRows + threadIdx.x;
        if (i < n) s[i] = fmaB(-alpha, v[i], r[i]);
    }
}

// After t = A s: partials t.s, t.t, s.s, rhat.s, rhat.t.
template <typename T, typename IT>
__global__ __launch_bounds__(kBlock) void bicg_split_st_w_kernel(const IterArgs<T, IT> *__restrict__ A) {
    A += blockIdx.y;  // system blockIdx.y of the launch
    if (load_done(A->st)) return;  // set by an earlier launch: uniform
    const int64_t n = A->n;
    const gptr<const T> s = glb((const T *)A->s);
    const gptr<const T> tv = glb((const T *)A->t);
    const gptr<const T> rh = glb((const T *)A->rh);
    double ts = 0.0, tt = 0.0, ss = 0.0, rs = 0.0, rt = 0.0;
    const TileRange tr = xcd_tiles(tiles_of(n));
    for (int64_t t = tr.first; t < tr.end; t += tr.stride) {
        const int64_t i = t * kTileRows + threadIdx.x;
        if (i >= n) continue;
        const T acc = tv[i], si = s[i], rhi = rh[i];
        ts = fma((double)acc, (double)si, ts);
        tt = fma((double)acc, (double)acc, tt);
        ss = fma((double)si, (double)si, ss);
        rs = fma((double)rhi, (double)si, rs);
        rt = fma((double)rhi, (double)acc, rt);
    }
    double red5[5] = {ts, tt, ss, rs, rt};
    const int slot[5] = {kBiTS, kBiTT, kBiSS, kBiRS, kBiRT};
    store_partials<5>(red5, A->part, slot);
}

// ------------------------------------------------------------------ launchers

// Row pairs: fp64 only (dia_tile never asks them for other types), and not
// on seven diagonals, where bicg_xpv's pairs (four vectors gathered at four
// offsets) need more than the 168 registers of three waves per SIMD and
// spill: those take the one-row fast tiles.
template <typename T>
bool bicg_pair(int cm, int tile, int slots) {
    return sizeof(T) == 8 && cm == kColDiaMajor && tile == kDiaTilePair && slots < 7;
}
#define SLA_BICG_O32(slots, ...)                                   \
    switch (slots) {                                               \
        case 3: { constexpr int kS = 3; __VA_ARGS__; } break;      \
        case 5: { constexpr int kS = 5; __VA_ARGS__; } break;      \
        default: { constexpr int kS = 7; __VA_ARGS__; } break;     \
    }
#define SLA_BICG_PAIR(slots, ...)                                  \
    switch (slots) {                                               \
        case 3: { constexpr int kS = 3; __VA_ARGS__; } break;      \
        default: { constexpr int kS = 5; __VA_ARGS__; } break;     \
    }

template <typename T, typename IT>
hipError_t launch_bicg_split(int part, const IterArgs<T, IT> *a, int64_t n, int nsys,
                             hipStream_t s) {
    const dim3 grid(grid_for_tiles(tiles_of(n)), nsys);
    switch (part) {
        case 0: bicg_split_xpv_u_kernel<T, IT><<<grid, kBlock, 0, s>>>(a); break;
        case 1: bicg_split_xpv_w_kernel<T, IT><<<grid, kBlock, 0, s>>>(a); break;
        case 2: bicg_split_st_u_kernel<T, IT><<<grid, kBlock, 0, s>>>(a); break;
        default: bicg_split_st_w_kernel<T, IT><<<grid, kBlock, 0, s>>>(a); break;
    }
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_bicg_init(int cm, const IterArgs<T, IT> *a, int64_t n, int nsys,
                            hipStream_t s) {
    // the iterations' grid: they read these partial sums
    bicg_init_kernel<T, IT><<<dim3(iter_grid(cm, 0, n), nsys), kBlock, 0, s>>>(a);
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_bicg_xpv(int slots, int cm, int tile, const IterArgs<T, IT> *a, int64_t n,
                           int nsys, hipStream_t s, const hipEvent_t *ev) {
    const dim3 grid(iter_grid(cm, 0, n), nsys);
    if (bicg_pair<T>(cm, tile, slots)) {
        if constexpr (sizeof(T) == 8)
            SLA_BICG_PAIR(slots, launch_maybe_timed(
                                     bicg_xpv_kernel<T, IT, kS, kColDiaMajor, true, true>, grid,
                                     dim3(kBlock), 0, s, ev, a));
    } else if (tile != kDiaTileGeneral && cm == kColDiaMajor) {
        SLA_BICG_O32(slots, launch_maybe_timed(bicg_xpv_kernel<T, IT, kS, kColDiaMajor, true>,
                                               grid, dim3(kBlock), 0, s, ev, a));
    } else {
        SLA_DISPATCH_FORM(cm, slots, launch_maybe_timed(bicg_xpv_kernel<T, IT, kS, kC>, grid,
                                                        dim3(kBlock), 0, s, ev, a));
    }
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_bicg_st(int slots, int cm, int tile, const IterArgs<T, IT> *a, int64_t n,
                          int nsys, hipStream_t s, const hipEvent_t *ev) {
    const dim3 grid(iter_grid(cm, 0, n), nsys);
    if (bicg_pair<T>(cm, tile, slots)) {
        if constexpr (sizeof(T) == 8)
            SLA_BICG_PAIR(slots, launch_maybe_timed(
                                     bicg_st_kernel<T, IT, kS, kColDiaMajor, true, true>, grid,
                                     dim3(kBlock), 0, s, ev, a));
    } else if (tile != kDiaTileGeneral && cm == kColDiaMajor) {
        SLA_BICG_O32(slots, launch_maybe_timed(bicg_st_kernel<T, IT, kS, kColDiaMajor, true>,
                                               grid, dim3(kBlock), 0, s, ev, a));
    } else {
        SLA_DISPATCH_FORM(cm, slots, launch_maybe_timed(bicg_st_kernel<T, IT, kS, kC>, grid,
                                                        dim3(kBlock), 0, s, ev, a));
    }
    return hipGetLastError();
}

#define SLA_INST(T, IT)                                                                        \
    template hipError_t launch_bicg_init<T, IT>(int, const IterArgs<T, IT> *, int64_t, int,    \
                                                hipStream_t);                                  \
    template hipError_t launch_bicg_xpv<T, IT>(int, int, int, const IterArgs<T, IT> *, int64_t, \
                                               int, hipStream_t, const hipEvent_t *);          \
    template hipError_t launch_bicg_st<T, IT>(int, int, int, const IterArgs<T, IT> *, int64_t, int, \
                                              hipStream_t, const hipEvent_t *);               \
    template hipError_t launch_bicg_split<T, IT>(int, const IterArgs<T, IT> *, int64_t, int,  \
                                                 hipStream_t);

SLA_INST(float, int32_t)
SLA_INST(float, int64_t)
SLA_INST(double, int32_t)
SLA_INST(double, int64_t)

}  // namespace sla
