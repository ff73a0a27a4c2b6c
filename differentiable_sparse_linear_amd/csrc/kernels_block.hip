// Conjugate gradients for small systems, one workgroup per system (torch-sla
// explainer, Methodology section 1: CG with the Jacobi preconditioner of the
// Significance section; the textbook recurrence, Saad, Iterative Methods for
// Sparse Linear Systems, Alg. 9.1, with z = M^-1 r).
//
// One workgroup (1024 threads, or 256 for at most 1024 rows) runs the whole
// solve of one small system (n <= 4096): vectors live in registers, the
// search direction in LDS for the gathers, reductions in LDS; no grid-wide
// synchronisation and no per-iteration launches (the pages note that launch
// overhead hurts iterative solvers on small problems: Problem statement,
// backend fragmentation).
#include "spmv_tile.h"

namespace sla {

template <typename T>
__device__ __forceinline__ T fmaT(T a, T b, T c) {
    return fma(a, b, c);
}

// Sum over a workgroup of NW wavefronts (16 or 4); every thread receives the
// same, order-fixed total.  Wavefront sums go to LDS; after the barrier,
// with 16 wavefronts lane l of every wavefront reads wavefront (l mod 16)'s
// sum and a 16-lane DPP row sum adds them (the same steps in every row of
// every wavefront); with 4, every lane reads the four sums and adds them in
// pairs.  Either way every thread gets bitwise the same total.
template <int NW, int NR>
__device__ __forceinline__ void block_sum(double (&v)[NR], double (*slots)[NW]) {
    static_assert(NW == 16 || NW == 4, "workgroups of 1024 or 256 threads");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const double w = wave_sum(v[r]);
        if (lane == 0) slots[r][wave] = w;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        if constexpr (NW == 16)
            v[r] = row16_sum(slots[r][lane & (NW - 1)]);
        else
            v[r] = (slots[r][0] + slots[r][1]) + (slots[r][2] + slots[r][3]);
    }
}

// One row's matrix entries, SLOTS slots (slots past the row repeat its last
// entry; they are left out of the sum).  The block path has n <= 4096, so an
// offset inside one system fits 32 bits and a column 16 bits.
template <typename T, int SLOTS>
__device__ __forceinline__ void block_row_load(gptr<const T> val, gptr<const int32_t> col, int lo,
                                               int len, T (&v)[SLOTS], int32_t (&c)[SLOTS]) {
    const int lastk = len > 0 ? len - 1 : 0;
#pragma unroll
    for (int k = 0; k < SLOTS; ++k) {
        const int idx = lo + (k < lastk ? k : lastk);
        v[k] = val[idx];
        c[k] = col[idx];
    }
}

// The row's product with the LDS-resident vector, in entry order; colf(k)
// gives slot k's column.
template <typename T, int SLOTS, typename CF>
__device__ __forceinline__ T block_row_dot(const T (&v)[SLOTS], CF colf, gptr<const T> val,
                                           gptr<const int32_t> col, const T *ps, int lo, int len) {
    T acc = T(0);
#pragma unroll
    for (int k = 0; k < SLOTS; ++k) {
        const T term = v[k] * ps[colf(k)];
        acc = k < len ? acc + term : acc;
    }
    for (int k = SLOTS; k < len; ++k) acc += val[lo + k] * ps[col[lo + k]];
    return acc;
}

// NT threads per workgroup (1024, or 256 for systems of at most 1024 rows).
// Row ownership: thread t owns rows t, t + NT, ... (RPT rows, interleaved so
// the vector accesses of a wavefront are consecutive).  The direction p
// lives in LDS, where every row's product gathers it, and so does x (read
// and written once per iteration); r, the row's own p and the product q of
// the owned rows stay in the thread's registers (each is read and written
// by its owner only), and so does M^-1 unless registers run short (fp64 with
// four rows per thread: then it is read from LDS twice per iteration, and
// without the resident matrix r and the row's own p are read from LDS too).
// An iteration touches LDS S + 3 (S + 5; S + 11) times per row: the S
// gathers of p, the store of the new p, x read and written (M^-1 read
// twice; r read twice and written, p read three times).  With RESIDENT
// (every row fits the slots) the thread's matrix entries are loaded once --
// values with the padding slots zeroed, columns packed two per register --
// and kept in registers for the whole solve, so the matrix is read from
// memory once per solve instead of once per iteration.  Otherwise the
// entries are re-read every iteration (the row offsets go through an empty
// asm so the compiler cannot hoist the address arithmetic out of the
// iteration loop).  Products: SLOTS slots per row, p gathered from LDS
// (neighbouring rows gather neighbouring LDS words), entry-order sums; rows
// longer than SLOTS finish with a loop.
// FULL: n == RPT * NT, every owned row exists, so the row
// loops carry no guard (a guard is a branch, and the compiler does not move
// the next row's LDS accesses above it).
template <typename T, typename IT, int NT, int RPT, int SLOTS, bool RESIDENT, bool FULL>
__global__ __launch_bounds__(NT) void block_cg_kernel(BlockCgParams P) {
    extern __shared__ unsigned char lds_raw[];
    const int64_t n = P.n, nnz = P.nnz;
    T *ps = reinterpret_cast<T *>(lds_raw);  // direction p (or x0 at the start)
    T *xs = ps + n;                          // iterate x
    T *ds = xs + n;                          // M^-1 (1 without preconditioner), when in LDS
    T *rs = ds + n;                          // r, when in LDS
    constexpr bool DREG = sizeof(T) == 4 || RPT <= 2;  // M^-1 in registers
    constexpr bool RREG = DREG || RESIDENT;            // r and own p in registers
    constexpr int NW = NT / 64;  // wavefronts per workgroup
    __shared__ double slots[4][3][NW];
    const int sys = blockIdx.x;
    const int tid = threadIdx.x;
    const gptr<const T> val = glb(reinterpret_cast<const T *>(P.val) + (int64_t)sys * nnz);
    const gptr<const T> b = glb(reinterpret_cast<const T *>(P.b) + (int64_t)sys * n);
    const gptr<T> x = glb(reinterpret_cast<T *>(P.x) + (int64_t)sys * n);
    const gptr<const IT> rp = glb(reinterpret_cast<const IT *>(P.rp));
    const gptr<const IT> dpos = glb(reinterpret_cast<const IT *>(P.diagpos));
    const gptr<const int32_t> col = glb(P.col);
    SolveState *st = P.st + sys;
    auto row_of = [&](int j) -> int { return tid + j * NT; };
    auto owned = [&](int i) -> bool { return FULL || i < n; };
    constexpr int MR = RESIDENT ? RPT : 1;
    constexpr int PC = (SLOTS + 1) / 2;
    constexpr int SR = RESIDENT ? 1 : RPT;

    int lo[SR], len[SR];  // row offsets (streaming mode only)
    T qr[RPT];            // product of the owned rows
    T pr_[RREG ? RPT : 1];  // p of the owned rows (RREG)
    T rr_[RREG ? RPT : 1];  // r of the owned rows (RREG)
    T dr[DREG ? RPT : 1];  // M^-1 of the owned rows (DREG)
    auto dinv = [&](int j, int i) -> T { return DREG ? dr[DREG ? j : 0] : ds[i]; };
    auto rget = [&](int j, int i) -> T { return RREG ? rr_[RREG ? j : 0] : rs[i]; };
    auto pget = [&](int j, int i) -> T { return RREG ? pr_[RREG ? j : 0] : ps[i]; };
    auto pset = [&](int j, int i, T v) {
        if (RREG) pr_[RREG ? j : 0] = v;
        ps[i] = v;
    };
    auto rset = [&](int j, int i, T v) {
        if (RREG)
            rr_[RREG ? j : 0] = v;
        else
            rs[i] = v;
    };
    T mv[MR][SLOTS];
    uint32_t mc[MR][PC];  // two 16-bit columns per register
    int bad = 0;
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int i = row_of(j);
        int l = 0, ln = 0;
        qr[j] = T(0);
        if (RREG) rr_[RREG ? j : 0] = pr_[RREG ? j : 0] = T(0);
        if (DREG) dr[DREG ? j : 0] = T(1);
        if (owned(i)) {
            l = (int)rp[i];
            ln = (int)(rp[i + 1] - rp[i]);
            const T x0 = P.use_x0 ? x[i] : T(0);
            xs[i] = x0;
            ps[i] = x0;
            T d = T(1);
            if (P.jac) {
                const T a = val[dpos[i]];
                bad |= (a == T(0));
                d = T(1) / a;
            }
            if (DREG)
                dr[DREG ? j : 0] = d;
            else
                ds[i] = d;
        }
        if (RESIDENT) {
            T v[SLOTS];
            int32_t c[SLOTS];
            block_row_load<T, SLOTS>(val, col, l, ln, v, c);
#pragma unroll
            for (int k = 0; k < SLOTS; ++k) mv[RESIDENT ? j : 0][k] = k < ln ? v[k] : T(0);
#pragma unroll
            for (int k = 0; k < PC; ++k)
                mc[RESIDENT ? j : 0][k] = (uint32_t)c[2 * k] |
                                          (2 * k + 1 < SLOTS ? (uint32_t)c[2 * k + 1] << 16 : 0u);
        } else {
            lo[RESIDENT ? 0 : j] = l;
            len[RESIDENT ? 0 : j] = ln;
        }
    }

    // out[j] = (A p)_i for the owned rows (p in LDS)
    auto spmv = [&](T(&out)[RPT]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            if (RESIDENT) {
                const uint32_t *pc = mc[RESIDENT ? j : 0];
                const T *v = mv[RESIDENT ? j : 0];
                T acc = T(0);
#pragma unroll
                for (int k = 0; k < SLOTS; ++k)
                    acc += v[k] * ps[(pc[k >> 1] >> (16 * (k & 1))) & 0xffffu];
                out[j] = acc;
            } else {
                int l = lo[RESIDENT ? 0 : j];
                asm volatile("" : "+v"(l));
                const int ln = len[RESIDENT ? 0 : j];
                T v[SLOTS];
                int32_t c[SLOTS];
                block_row_load<T, SLOTS>(val, col, l, ln, v, c);
                out[j] = block_row_dot<T, SLOTS>(v, [&](int k) { return c[k]; }, val, col, ps, l, ln);
            }
        }
    };

    __syncthreads();
    if (P.use_x0) spmv(qr);  // A x0 (ps holds x0)
    double r0[3] = {0.0, 0.0, 0.0};  // r.z, r.r, b.b
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int i = row_of(j);
        if (owned(i)) {
            const T bi = b[i];
            const T ri = P.use_x0 ? bi - qr[j] : bi;
            rset(j, i, ri);
            const T zi = dinv(j, i) * ri;
            r0[0] += (double)ri * (double)zi;
            r0[1] += (double)ri * (double)ri;
            r0[2] += (double)bi * (double)bi;
        }
    }
    block_sum<NW>(r0, slots[0]);  // its barrier also ends every read of x0 in ps
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int i = row_of(j);
        if (owned(i)) pset(j, i, dinv(j, i) * rget(j, i));  // p_0 = z_0
    }
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
            spmv(qr);
            double pq[1] = {0.0};
#pragma unroll
            for (int j = 0; j < RPT; ++j) {
                const int i = row_of(j);
                if (owned(i)) pq[0] += (double)pget(j, i) * (double)qr[j];
            }
            block_sum<NW>(pq, slots[slot]);  // every gather of p is done
            slot = (slot + 1) & 3;
            if (!(pq[0] > 0.0)) {
                status = SLA_BREAKDOWN;
                break;
            }
            const T alpha = (T)(rho / pq[0]);
            double red[2] = {0.0, 0.0};
#pragma unroll
            for (int j = 0; j < RPT; ++j) {
                const int i = row_of(j);
                if (owned(i)) {
                    xs[i] = fmaT(alpha, pget(j, i), xs[i]);
                    const T ri = fmaT(-alpha, qr[j], rget(j, i));
                    rset(j, i, ri);
                    const T zi = dinv(j, i) * ri;
                    red[0] += (double)ri * (double)zi;
                    red[1] += (double)ri * (double)ri;
                }
            }
            block_sum<NW>(red, slots[slot]);
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
            for (int j = 0; j < RPT; ++j) {
                const int i = row_of(j);
                if (owned(i)) pset(j, i, fmaT(beta, pget(j, i), dinv(j, i) * rget(j, i)));
            }
            __syncthreads();  // the new p is complete before the next product
        }
    }
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int i = row_of(j);
        if (owned(i)) x[i] = zero_x ? T(0) : xs[i];
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

// ------------------------------------------------------------------ launcher

// The matrix stays in registers when every row fits the slots and a
// thread's entries fit in 56 VGPRs.
template <typename T, int RPT, int SLOTS>
constexpr bool block_resident() {
    return RPT * (SLOTS * ((int)sizeof(T) / 4) + (SLOTS + 1) / 2) <= 56;
}

// Slots per row for the block solver: the longest row rounded up to 4, 5, 6
// or 8 (5 is the five-point stencil's exact width); longer rows stream.
// Systems of at most kBlockSmallN rows take 256-thread workgroups (up to four
// rows per thread), larger ones 1024 threads.  Every thread runs the
// iteration's reductions and scalar steps whatever its row count, so for a
// small system four wavefronts issue a quarter of the instructions that
// sixteen would; batches of small systems also fit several workgroups per
// compute unit.
constexpr int64_t kBlockSmallN = 1024;

template <typename T, typename IT>
hipError_t launch_block_cg(int max_len, const BlockCgParams &p, int batch, hipStream_t s) {
    const size_t lds = 4 * (size_t)p.n * sizeof(T);  // p, x, M^-1, r
    const bool small = p.n <= kBlockSmallN;
    const int nt = small ? 256 : kBlockSolveThreads;
    const int rpt = (int)((p.n + nt - 1) / nt);
    const bool fits = max_len <= 8;
#define SLA_BLOCK_LAUNCH(N, R, S)                                                                  \
    if (fits && block_resident<T, R, S>() && p.n == R * N)                                        \
        block_cg_kernel<T, IT, N, R, S, block_resident<T, R, S>(), true>                           \
            <<<batch, N, lds, s>>>(p);                                                             \
    else if (fits && block_resident<T, R, S>())                                                    \
        block_cg_kernel<T, IT, N, R, S, block_resident<T, R, S>(), false>                          \
            <<<batch, N, lds, s>>>(p);                                                             \
    else                                                                                           \
        block_cg_kernel<T, IT, N, R, S, false, false><<<batch, N, lds, s>>>(p)
#define SLA_BLOCK_ROWS(N, R)                  \
    if (max_len <= 4) {                       \
        SLA_BLOCK_LAUNCH(N, R, 4);            \
    } else if (max_len == 5) {                \
        SLA_BLOCK_LAUNCH(N, R, 5);            \
    } else if (max_len == 6) {                \
        SLA_BLOCK_LAUNCH(N, R, 6);            \
    } else {                                  \
        SLA_BLOCK_LAUNCH(N, R, 8);            \
    }
    if (small) {
        if (rpt <= 1) {
            SLA_BLOCK_ROWS(256, 1)
        } else if (rpt <= 2) {
            SLA_BLOCK_ROWS(256, 2)
        } else {
            SLA_BLOCK_ROWS(256, 4)
        }
    } else if (rpt <= 2) {  // n > 1024: at least two rows per thread
        SLA_BLOCK_ROWS(kBlockSolveThreads, 2)
    } else {
        SLA_BLOCK_ROWS(kBlockSolveThreads, 4)
    }
#undef SLA_BLOCK_ROWS
#undef SLA_BLOCK_LAUNCH
    return hipGetLastError();
}

#define SLA_INST(T, IT) \
    template hipError_t launch_block_cg<T, IT>(int, const BlockCgParams &, int, hipStream_t);

SLA_INST(float, int32_t)
SLA_INST(float, int64_t)
SLA_INST(double, int32_t)
SLA_INST(double, int64_t)

}  // namespace sla
