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

// System blockIdx.y's values: val + y * val_stride, or, for a solver's
// product (ind not null), those its argument block names.
template <typename T, typename IT>
__device__ __forceinline__ const T *sys_values(const T *val, int64_t val_stride,
                                               const IterArgs<T, IT> *ind) {
    return ind ? ind[blockIdx.y].val : val + (int64_t)blockIdx.y * val_stride;
}

// A solver's product has nothing to do once its system has stopped (set by
// an earlier launch, so every wavefront reads the same).
template <typename T, typename IT>
__device__ __forceinline__ bool sys_stopped(const IterArgs<T, IT> *ind) {
    return ind && load_done(ind[blockIdx.y].st);
}

// s + a * b with the product rounded before the addition (no fused
// multiply-add): the terms of A^T g are formed this way on every path, so
// that the paths agree bit for bit.
template <typename T>
__device__ __forceinline__ T add_product(T s, T a, T b) {
#pragma clang fp contract(off)
    return s + a * b;
}

template <typename T, typename IT, int SLOTS, int CM>
__global__ __launch_bounds__(kBlock) void spmv_kernel(const IT *__restrict__ rp, ColArgs ca,
                                                      const T *__restrict__ val, int64_t val_stride,
                                                      const T *__restrict__ x, T *__restrict__ y,
                                                      int64_t n, int64_t vec_stride,
                                                      const uint8_t *plan_tiles,
                                                      const IterArgs<T, IT> *ind) {
    if (sys_stopped(ind)) return;
    __shared__ RowLds<T, IT> sm;
    const int sys = blockIdx.y;
    const gptr<const T> v = glb(sys_values(val, val_stride, ind));
    const gptr<const T> xs = glb(x + (int64_t)sys * vec_stride);
    const gptr<T> ys = glb(y + (int64_t)sys * vec_stride);
    spmv_rows<T, IT, SLOTS, SLOTS>(
        xcd_tiles(tiles_of(n)), n, glb(rp), col_src<CM>(ca), sm, [&](IT k) { return v[k]; },
        [&](int32_t c) { return xs[c]; }, PlainGather(), NoOwn(),
        [&](int64_t i, T s, int, T) { ys[i] = s; }, NoPre(), NoPost(), plan_tiles);
}

// Backward pass of y = A x on a pattern with per-row diagonal masks, one row
// i per thread, reading A's own rows (no transpose map):
//  GX: gx[i] = (A^T g)_i.  Row i of A^T holds A[j][i] for j = i - dlt[q],
//      stored when bit q of msk[j] is set, at position rp[j] + (set bits of
//      msk[j] below q).  q runs downwards, so the terms A[j][i] g_j (each
//      rounded, then added, from 0) are added in ascending j, the column
//      order of A^T's row: the sums of rowsum_kernel.  All NDT slots are
//      unrolled so every mask and row-pointer load of a row is in flight
//      before its values are gathered.
//  GV: gv[k] = g_i x_j for row i's stored entries (NEG: -g_i x_j, the
//      solve's gradient on the pattern with g = lambda).  Entry k = rp[i] +
//      (set bits of msk[i] below q) has column i + dlt[q], so the x loads of
//      one diagonal are consecutive across the wavefront.  The products go
//      to LDS at the entry's place in the tile's run (at most 8 entries per
//      row in this form, so a tile's run fits kCap) and leave as one
//      coalesced run: a row's entries lie 8 bytes apart, and stores straight
//      from the rows would scatter each store instruction over many lines.
//      The run is stored non-temporally (written once, not read here; on
//      the 1e6-row 3D diffusion system 17.3 -> 14.3 us, at 512^3 3.23 ->
//      3.05 ms).
// NDT >= the pattern's diagonal count.  System blockIdx.y: values
// val + y * val_stride, vectors + y * n, gv + y * nnz.
template <typename T, typename IT, int NDT, bool GX, bool GV, bool NEG>
__global__ __launch_bounds__(kBlock) void diag_vjp_kernel(const IT *__restrict__ rp, ColArgs ca,
                                                          const T *__restrict__ val,
                                                          int64_t val_stride,
                                                          const T *__restrict__ g,
                                                          const T *__restrict__ x,
                                                          T *__restrict__ gx,
                                                          T *__restrict__ gv, int64_t n,
                                                          int64_t nnz) {
    const int sys = blockIdx.y;
    const gptr<const T> v = glb(GX ? val + (int64_t)sys * val_stride : val);
    const gptr<const T> gs = glb(g + (int64_t)sys * n);
    const gptr<const T> xs = glb(GV ? x + (int64_t)sys * n : x);
    const gptr<T> gxs = glb(GX ? gx + (int64_t)sys * n : gx);
    const gptr<T> gvs = glb(GV ? gv + (int64_t)sys * nnz : gv);
    const gptr<const uint16_t> msk = glb(ca.msk);
    const gptr<const IT> rpg = glb(rp);
    const int nd = ca.nd;
    int32_t dl[NDT];
#pragma unroll
    for (int q = 0; q < NDT; ++q) dl[q] = q < nd ? ca.dlt[q] : 0;
    __shared__ T sg[GV ? kCap : 1];
    const TileRange tr = xcd_tiles(tiles_of(n));
    for (int64_t t = tr.first; t < tr.end; t += tr.stride) {
        const int64_t row0 = t * kTileRows;
        const int64_t i = row0 + threadIdx.x;
        if constexpr (GV) {
            const int rows = n - row0 < kTileRows ? (int)(n - row0) : kTileRows;
            const IT base = rpg[row0];
            const int cnt = (int)(rpg[row0 + rows] - base);
            if (i < n) {
                const uint32_t m = msk[i];
                const int at = (int)(rpg[i] - base);
                const T gi = gs[i];
#pragma unroll
                for (int q = 0; q < NDT; ++q) {
                    if (q < nd && ((m >> q) & 1u)) {
                        const T pr = gi * xs[i + dl[q]];
                        sg[at + __builtin_popcount(m & ((1u << q) - 1u))] = NEG ? -pr : pr;
                    }
                }
            }
            __syncthreads();
            for (int e = threadIdx.x; e < cnt; e += kBlock)
                __builtin_nontemporal_store(sg[e], &gvs[base + e]);
            __syncthreads();  // the next tile reuses sg
        }
        if (i >= n) continue;
        if constexpr (GX) {
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
                if (on[q]) s = add_product(s, v[k[q]], gs[jj[q]]);
            }
            gxs[i] = s;
        }
    }
}

// One pass over A's entries by row, entry k of row i (g = g[i]), writing
// one of:
//  GV: the gradient on the pattern, grad[k] = g x[col[k]] (NEG: -lambda_i
//      x_j, the solve's gradient with g = lambda; else the product's);
//  SC: the terms of A^T g, c[pinv[k]] = val[k] g, each written to entry k's
//      place among A^T's entries (pinv: A's entry -> A^T's), so that a
//      second pass (rowsum_kernel) sums every row of A^T over consecutive
//      memory.  The values are read in A's order, coalesced; the writes land
//      at scattered 8-byte places, where reading val[perm[kt]] row by row of
//      A^T would fetch a whole line per entry.
// (Both in one pass measured slower than the two passes: the scattered
// partial-line writes and the gradient's streaming writes contend.)  The
// gradient is stored non-temporally: written once and not read here, it
// would otherwise push the scattered terms and the inputs of the next pass
// out of the Infinity Cache (measured on a 2^20-row power-law graph, the
// backward pass with both outputs: 258 us with plain stores, 168 us with
// these).  plan_grad_kernel stores it the same way.
// Per-entry column forms (int32 or tile-relative int16; diagonal masks use
// diag_vjp_kernel).  Short tiles: each thread marks the tile-local row of its
// row's entries in LDS, then the entries go as one coalesced run.  Tiles
// that plan_tiles flags are left to the row plan; other tiles past the stage
// take one wavefront per row.  System blockIdx.y: g, x + y * n; grad, val,
// c + y * nnz.
template <typename T, typename IT, bool NEG, int CM, bool GV, bool SC>
__global__ __launch_bounds__(kBlock) void grad_kernel(const IT *__restrict__ rp, ColArgs ca,
                                                      const T *__restrict__ g,
                                                      const T *__restrict__ x, T *__restrict__ grad,
                                                      const T *__restrict__ val,
                                                      const int32_t *__restrict__ pinv,
                                                      T *__restrict__ c, int64_t n, int64_t nnz,
                                                      const uint8_t *plan_tiles) {
    static_assert(CM == kColWide || CM == kColTile16, "per-entry column forms");
    static_assert(GV != SC, "one of the two outputs");
    __shared__ IT srp[kTileRows + 1];
    __shared__ T sg[kTileRows];
    __shared__ uint16_t rid[kCap];
    const int sys = blockIdx.y;
    const ColSrc<CM> col = col_src<CM>(ca);
    const gptr<const T> gs = glb(g + (int64_t)sys * n);
    const gptr<const T> xs = glb(GV ? x + (int64_t)sys * n : x);
    const gptr<T> gr = glb(GV ? grad + (int64_t)sys * nnz : grad);
    const gptr<const T> vs = glb(SC ? val + (int64_t)sys * nnz : val);
    const gptr<T> cs = glb(SC ? c + (int64_t)sys * nnz : c);
    const gptr<const int32_t> pv = glb(pinv);
    const int tid = threadIdx.x;
    const TileRange tr = xcd_tiles(tiles_of(n));
    for (int64_t t = tr.first; t < tr.end; t += tr.stride) {
        const int64_t row0 = t * kTileRows;
        const int64_t left = n - row0;
        const int rows = left < kTileRows ? (int)left : kTileRows;
        if (tid < rows) {
            srp[tid] = rp[row0 + tid];
            sg[tid] = gs[row0 + tid];
        }
        if (tid == 0) srp[rows] = rp[row0 + rows];
        __syncthreads();
        const IT base = srp[0];
        const int64_t cnt = (int64_t)(srp[rows] - base);
        const bool planned = plan_tiles && plan_tiles[t];
        if (!planned && cnt <= kCap) {
            if (tid < rows) {
                for (int e = (int)(srp[tid] - base); e < (int)(srp[tid + 1] - base); ++e)
                    rid[e] = (uint16_t)tid;
            }
            __syncthreads();
            int32_t cj[kEpt], pj[kEpt];
            T vj[kEpt];
#pragma unroll
            for (int j = 0; j < kEpt; ++j) {
                const int e = tid + j * kBlock;
                if (e < cnt) {
                    if constexpr (GV) cj[j] = col(base + e, row0);
                    if constexpr (SC) {
                        vj[j] = vs[base + e];
                        pj[j] = pv[base + e];
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < kEpt; ++j) {
                const int e = tid + j * kBlock;
                if (e < cnt) {
                    const T gi = sg[rid[e]];
                    if constexpr (GV) {
                        const T p = gi * xs[cj[j]];
                        __builtin_nontemporal_store(NEG ? -p : p, &gr[base + e]);
                    }
                    if constexpr (SC) {
                        if ((uint32_t)pj[j] < (uint64_t)nnz) cs[pj[j]] = vj[j] * gi;
                    }
                }
            }
        } else if (!planned) {
            const int lane = tid & 63, wave = tid >> 6;
            for (int r = wave; r < rows; r += kWaves) {
                const T gi = sg[r];
                const IT lo = srp[r], hi = srp[r + 1];
                for (IT k = lo + lane; k < hi; k += 64) {
                    if constexpr (GV) {
                        const T p = gi * xs[col(k, row0)];
                        __builtin_nontemporal_store(NEG ? -p : p, &gr[k]);
                    }
                    if constexpr (SC) {
                        const int32_t q = pv[k];
                        if ((uint32_t)q < (uint64_t)nnz) cs[q] = vs[k] * gi;
                    }
                }
            }
        }
        __syncthreads();
    }
}

// y = A^T g summed row by row of A^T (rp: A^T's row pointers), each row's
// terms A_ij g_i in entry order (ascending i), each rounded, then added from
// 0.  The terms come from
//  - !PERM: the scatter pass (grad_kernel / plan_grad_kernel with SC), which
//    left them in A^T's order in t (one system per blockIdx.y, nnz apart);
//  - PERM: A^T's values through the transpose map, t[perm[k]] * g[col[k]]
//    (col: A^T's columns; values val_stride apart, g and y n apart), the
//    form for a batch of systems in one launch.
// A tile's terms are staged in LDS as one run, then thread t adds row t's
// one after another (the order and the rounding of the row plan's short
// blocks).  With lidx (!PERM) the staged tiles' terms are in A's entry
// order in t and go to their places in A^T's order in LDS (lidx[k]: the
// offset in the tile of the term at k; setup_buckets).  Tiles that
// plan_tiles flags are left to the row plan (whose short blocks honour lidx
// the same way); other tiles past the stage take one wavefront per row
// (lane-strided partial sums, then a fixed-order wavefront sum).
template <typename T, typename IT, bool PERM>
__global__ __launch_bounds__(kBlock) void rowsum_kernel(const IT *__restrict__ rp,
                                                        const T *__restrict__ t,
                                                        int64_t t_stride,
                                                        const int32_t *__restrict__ perm,
                                                        const int32_t *__restrict__ col,
                                                        const T *__restrict__ g,
                                                        T *__restrict__ y, int64_t n,
                                                        const uint8_t *plan_tiles,
                                                        const uint16_t *__restrict__ lidx) {
    __shared__ IT srp[kTileRows + 1];
    __shared__ T sc[kCap];
    const int sys = blockIdx.y;
    const gptr<const T> ts = glb(t + (int64_t)sys * t_stride);
    const gptr<const T> gs = glb(PERM ? g + (int64_t)sys * n : g);
    const gptr<const int32_t> pm = glb(perm);
    const gptr<const int32_t> cl = glb(col);
    const gptr<T> ys = glb(y + (int64_t)sys * n);
    const int tid = threadIdx.x;
    const TileRange tr = xcd_tiles(tiles_of(n));
    for (int64_t tt = tr.first; tt < tr.end; tt += tr.stride) {
        const int64_t row0 = tt * kTileRows;
        const int64_t left = n - row0;
        const int rows = left < kTileRows ? (int)left : kTileRows;
        if (plan_tiles && plan_tiles[tt]) continue;  // the same in the whole workgroup
        if (tid < rows) srp[tid] = rp[row0 + tid];
        if (tid == 0) srp[rows] = rp[row0 + rows];
        __syncthreads();
        const IT base = srp[0];
        const int64_t cnt = (int64_t)(srp[rows] - base);
        if (cnt <= kCap) {
            T v[kEpt];
            if constexpr (PERM) {
                int32_t pj[kEpt], cj[kEpt];
#pragma unroll
                for (int j = 0; j < kEpt; ++j) {
                    const int e = tid + j * kBlock;
                    pj[j] = e < cnt ? pm[base + e] : 0;
                    cj[j] = e < cnt ? cl[base + e] : 0;
                }
#pragma unroll
                for (int j = 0; j < kEpt; ++j) {
                    const int e = tid + j * kBlock;
                    v[j] = e < cnt ? ts[pj[j]] * gs[cj[j]] : T(0);
                }
            } else if (lidx) {
                int dst[kEpt];
#pragma unroll
                for (int j = 0; j < kEpt; ++j) {
                    const int e = tid + j * kBlock;
                    v[j] = e < cnt ? ts[base + e] : T(0);
                    dst[j] = e < cnt ? (int)lidx[base + e] & (kCap - 1) : -1;
                }
#pragma unroll
                for (int j = 0; j < kEpt; ++j)
                    if (dst[j] >= 0) sc[dst[j]] = v[j];
            } else {
#pragma unroll
                for (int j = 0; j < kEpt; ++j) {
                    const int e = tid + j * kBlock;
                    v[j] = e < cnt ? ts[base + e] : T(0);
                }
            }
            if (PERM || !lidx) {
#pragma unroll
                for (int j = 0; j < kEpt; ++j) sc[tid + j * kBlock] = v[j];
            }
            __syncthreads();
            if (tid < rows) {
                const int hi = (int)(srp[tid + 1] - base);
                T s = T(0);
                for (int e = (int)(srp[tid] - base); e < hi; ++e) s += sc[e];
                ys[row0 + tid] = s;
            }
        } else {
            const int lane = tid & 63, wave = tid >> 6;
            for (int r = wave; r < rows; r += kWaves) {
                T s = T(0);
                for (IT k = srp[r] + lane; k < srp[r + 1]; k += 64) {
                    if constexpr (PERM)
                        s = add_product(s, ts[pm[k]], gs[cl[k]]);
                    else
                        s += ts[k];
                }
                s = wave_sum_t(s);
                if (lane == 0) ys[row0 + r] = s;
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------ row plans
//
// The tiles past the stage (PlanItem): workgroup b takes item b, system
// blockIdx.y (values val_stride apart, vectors vec_stride apart, partials
// nslots apart).  MODE kPlanA: the operator's own values; kPlanPerm: A^T
// through the transpose map, entry k's value val[perm[k]]; kPlanSum: the
// row sums of val alone (rowsum_kernel's rows past the stage; x unused).
// The A^T modes round every term before adding it, as rowsum_kernel does.
constexpr int kPlanA = 0, kPlanPerm = 1, kPlanSum = 2;

// Products of one item.  Short block: the run's products v x[col] go to
// LDS in one coalesced pass (kPlanSum with lidx: the terms the scatter pass
// wrote in A's entry order, each to its offset lidx[k] in A^T's order),
// then thread t adds row r0 + t's products in entry order.  Long-row chunk: thread t takes entries t, t + 256, ... of
// the chunk (all loads first, then an fma chain), a fixed-order workgroup
// sum, y[row] or the chunk's partial.
template <typename T, typename IT, int MODE>
__global__ __launch_bounds__(kBlock) void plan_spmv_kernel(
    const PlanItem *__restrict__ items, const IT *__restrict__ rp, const int32_t *__restrict__ col,
    const int32_t *__restrict__ perm, const T *__restrict__ val, int64_t val_stride,
    const T *__restrict__ x, T *__restrict__ y, int64_t vec_stride, T *__restrict__ part,
    int32_t nslots, const IterArgs<T, IT> *ind, const uint16_t *__restrict__ lidx) {
    static_assert((kPlanCap & (kPlanCap - 1)) == 0, "lidx offsets are masked to the block");
    if (sys_stopped(ind)) return;
    __shared__ T prod[kPlanCap];
    __shared__ T wsum[kWaves];
    const int sys = blockIdx.y;
    const gptr<const T> v = glb(sys_values(val, val_stride, ind));
    const gptr<const T> xs = glb(MODE == kPlanSum ? x : x + (int64_t)sys * vec_stride);
    const gptr<T> ys = glb(y + (int64_t)sys * vec_stride);
    const gptr<const int32_t> cg = glb(col);
    const gptr<const int32_t> pm = glb(perm);
    auto vf = [&](int64_t k) { return MODE == kPlanPerm ? v[pm[k]] : v[k]; };
    const PlanItem it = items[blockIdx.x];
    const int tid = threadIdx.x;
    const int64_t e0 = it.e0;
    const int cnt = (int)(it.e1 - e0);
    T pv[kPlanEpt], px[kPlanEpt];
#pragma unroll
    for (int j = 0; j < kPlanEpt; ++j) {
        const int e = tid + j * kBlock;
        pv[j] = T(0);
        px[j] = T(0);
        if (e < cnt) {
            pv[j] = vf(e0 + e);
            px[j] = MODE == kPlanSum ? T(1) : xs[cg[e0 + e]];
        }
    }
    if (it.kind == 0) {
        if (MODE == kPlanSum && lidx) {  // terms in A's order: back to A^T's
            int dst[kPlanEpt];
#pragma unroll
            for (int j = 0; j < kPlanEpt; ++j) {
                const int e = tid + j * kBlock;
                dst[j] = e < cnt ? (int)lidx[e0 + e] & (kPlanCap - 1) : -1;
            }
#pragma unroll
            for (int j = 0; j < kPlanEpt; ++j)
                if (dst[j] >= 0) prod[dst[j]] = pv[j] * px[j];
        } else {
#pragma unroll
            for (int j = 0; j < kPlanEpt; ++j) {
                const int e = tid + j * kBlock;
                if (e < cnt) prod[e] = pv[j] * px[j];
            }
        }
        __syncthreads();
        if (tid < it.r1 - it.r0) {
            const int64_t r = it.r0 + tid;
            const int lo = (int)(rp[r] - e0), hi = (int)(rp[r + 1] - e0);
            T s = T(0);
            for (int k = lo; k < hi; ++k) s += prod[k];
            ys[r] = s;
        }
    } else {
        T s = T(0);
#pragma unroll
        for (int j = 0; j < kPlanEpt; ++j)  // 0 * 0 past the chunk
            s = MODE == kPlanA ? fma(pv[j], px[j], s) : add_product(s, pv[j], px[j]);
        s = wave_sum_t(s);
        if ((tid & 63) == 0) wsum[tid >> 6] = s;
        __syncthreads();
        if (tid == 0) {
            T tot = T(0);
#pragma unroll
            for (int w = 0; w < kWaves; ++w) tot += wsum[w];
            if (it.slot < 0)
                ys[it.r0] = tot;
            else
                part[(int64_t)sys * nslots + it.slot] = tot;
        }
    }
}

// A split row's value from its chunks' partials, one wavefront per split
// row: lane l adds partials l, l + 64, ... in order, then a fixed-order
// wavefront sum.
template <typename T, typename IT>
__global__ __launch_bounds__(kBlock) void plan_finish_kernel(const PlanFin *__restrict__ fin,
                                                             int32_t nfin,
                                                             const T *__restrict__ part,
                                                             int32_t nslots, T *__restrict__ y,
                                                             int64_t vec_stride,
                                                             const IterArgs<T, IT> *ind) {
    if (sys_stopped(ind)) return;
    const int sys = blockIdx.y;
    const int f = blockIdx.x * kWaves + (threadIdx.x >> 6);  // the same in the whole wavefront
    if (f >= nfin) return;
    const int lane = threadIdx.x & 63;
    const PlanFin r = fin[f];
    const T *p = part + (int64_t)sys * nslots + r.slot0;
    T s = T(0);
    for (int c = lane; c < r.nch; c += 64) s += p[c];
    s = wave_sum_t(s);
    if (lane == 0) y[(int64_t)sys * vec_stride + r.row] = s;
}

// grad_kernel's pass (GV, SC, NEG as there) for one item.  Short block:
// thread t marks row r0 + t's entries in LDS, then the run goes coalesced;
// long-row chunk: one row, coalesced.
template <typename T, typename IT, bool NEG, bool GV, bool SC>
__global__ __launch_bounds__(kBlock) void plan_grad_kernel(
    const PlanItem *__restrict__ items, const IT *__restrict__ rp, const int32_t *__restrict__ col,
    const T *__restrict__ g, const T *__restrict__ x, T *__restrict__ grad,
    const T *__restrict__ val, const int32_t *__restrict__ pinv, T *__restrict__ c, int64_t n,
    int64_t nnz, int32_t nitems) {
    static_assert(GV != SC, "one of the two outputs");
    __shared__ uint16_t rid[kPlanCap];
    __shared__ T sg[kTileRows];
    // each XCD takes a contiguous range of items (workgroups go to the XCDs
    // in turn), so the scatter pass's writes to one tile of A^T (pinv: the
    // handle's bpos) come from one XCD in runs of consecutive addresses
    const int per = (int)gridDim.x / kNumXcd;
    const int64_t item = (int64_t)(blockIdx.x % kNumXcd) * per + blockIdx.x / kNumXcd;
    if (item >= nitems) return;
    const int sys = blockIdx.y;
    const gptr<const T> gs = glb(g + (int64_t)sys * n);
    const gptr<const T> xs = glb(GV ? x + (int64_t)sys * n : x);
    const gptr<T> gr = glb(GV ? grad + (int64_t)sys * nnz : grad);
    const gptr<const T> vs = glb(SC ? val + (int64_t)sys * nnz : val);
    const gptr<T> cs = glb(SC ? c + (int64_t)sys * nnz : c);
    const gptr<const int32_t> pv = glb(pinv);
    const gptr<const int32_t> cg = glb(col);
    const PlanItem it = items[item];
    const int tid = threadIdx.x;
    const int64_t e0 = it.e0;
    const int cnt = (int)(it.e1 - e0);
    const bool block = it.kind == 0;
    if (block) {
        if (tid < it.r1 - it.r0) {
            const int64_t r = it.r0 + tid;
            sg[tid] = gs[r];
            const int hi = (int)(rp[r + 1] - e0);
            for (int e = (int)(rp[r] - e0); e < hi; ++e) rid[e] = (uint16_t)tid;
        }
        __syncthreads();
    }
    const T g0 = block ? T(0) : gs[it.r0];
    int32_t cj[kPlanEpt], pj[kPlanEpt];
    T vj[kPlanEpt];
#pragma unroll
    for (int j = 0; j < kPlanEpt; ++j) {
        const int e = tid + j * kBlock;
        if (e < cnt) {
            if constexpr (GV) cj[j] = cg[e0 + e];
            if constexpr (SC) {
                vj[j] = vs[e0 + e];
                pj[j] = pv[e0 + e];
            }
        }
    }
#pragma unroll
    for (int j = 0; j < kPlanEpt; ++j) {
        const int e = tid + j * kBlock;
        if (e < cnt) {
            const T gi = block ? sg[rid[e]] : g0;
            if constexpr (GV) {
                const T p = gi * xs[cj[j]];
                __builtin_nontemporal_store(NEG ? -p : p, &gr[e0 + e]);
            }
            if constexpr (SC) {
                if ((uint32_t)pj[j] < (uint64_t)nnz) cs[pj[j]] = vj[j] * gi;
            }
        }
    }
}

// out[pinv[k]] = val[k]: the values in A^T's entry order, read coalesced.
// (Here and in the scatter pass a position outside [0, nnz), which only a
// faulty map could hold, is skipped rather than written.)
template <typename T>
__global__ __launch_bounds__(kBlock) void scatter_kernel(const int32_t *__restrict__ pinv,
                                                         const T *__restrict__ val,
                                                         T *__restrict__ out, int64_t nnz) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x; k < nnz; k += stride)
        if ((uint32_t)pinv[k] < (uint64_t)nnz) out[pinv[k]] = val[k];
}

// Bit-for-bit equality (a signed zero differs from an unsigned one, a NaN
// from everything).
template <typename T>
__device__ __forceinline__ bool same_bits(T a, T b) {
    if constexpr (sizeof(T) == 8)
        return __builtin_bit_cast(uint64_t, a) == __builtin_bit_cast(uint64_t, b);
    else
        return __builtin_bit_cast(uint32_t, a) == __builtin_bit_cast(uint32_t, b);
}

// out[q * n + i] = row i's entry on diagonal q, 0 where bit q of msk[i] is
// clear.  The row's entries are stored in ascending column order, which is
// ascending q, so the k-th set bit takes the k-th entry.  System blockIdx.y
// reads val + y * val_stride and writes out + y * nd * n.  With st (mirrored
// offsets), row i's entry on a diagonal q below the main one is compared
// with the entry of row j = i + off[q] on the mirrored diagonal nd-1-q
// (column i): both present and equal in every bit, or both absent; any other
// outcome sets st[y].asym.  Every pair of mirrored positions is the lower
// position of exactly one row, so the check covers the whole matrix.
template <typename T, typename IT>
__global__ __launch_bounds__(kBlock) void dia_pack_kernel(const IT *__restrict__ rp,
                                                          const ColArgs cols,
                                                          const T *__restrict__ val,
                                                          int64_t val_stride,
                                                          T *__restrict__ out, int64_t n,
                                                          SolveState *st) {
    const uint16_t *__restrict__ msk = cols.msk;
    const int nd = cols.nd;
    val += (int64_t)blockIdx.y * val_stride;
    out += (int64_t)blockIdx.y * nd * n;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    int bad = 0;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride) {
        const uint32_t mi = msk[i];
        uint32_t m = mi;
        IT k = rp[i];
        for (int q = 0; q < nd; ++q, m >>= 1) {
            T v = T(0);
            if (m & 1u) v = val[k++];
            out[(int64_t)q * n + i] = v;
            if (st && 2 * q + 1 < nd) {
                const int64_t j = i + cols.off[q];
                const uint32_t mj = j >= 0 ? msk[j] : 0u;
                const int qm = nd - 1 - q;
                const bool hi = (mi >> q) & 1u, hj = (mj >> qm) & 1u;
                if (hi != hj)
                    bad = 1;
                else if (hi)
                    bad |= !same_bits(v, val[rp[j] + __builtin_popcount(mj & ((1u << qm) - 1u))]);
            }
        }
    }
    if (st) raise_flag(bad, &st[blockIdx.y].asym);
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

// *poll = *ndone, stored at system scope into pinned host memory: once the
// stream has passed this kernel the host reads the count of stopped systems
// without a copy of its own.
__global__ __launch_bounds__(64) void publish_kernel(const int32_t *ndone, int32_t *poll) {
    if (threadIdx.x == 0)
        __hip_atomic_store(poll, *ndone, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// ------------------------------------------------------------------ launchers

inline bool planned(const RowPlan *plan) { return plan && plan->nitems > 0; }

// The plan's rows of y = A x (MODE as for plan_spmv_kernel), after the tile
// kernel has done the others.
template <typename T, typename IT, int MODE>
void launch_plan_spmv(const RowPlan &pl, const IT *rp, const int32_t *perm, const T *val,
                      int64_t val_stride, const T *x, T *y, int64_t vec_stride, int batch,
                      hipStream_t s, const IterArgs<T, IT> *ind = nullptr,
                      const uint16_t *lidx = nullptr) {
    T *part = reinterpret_cast<T *>(pl.part);
    plan_spmv_kernel<T, IT, MODE><<<dim3(pl.nitems, batch), kBlock, 0, s>>>(
        pl.items, rp, pl.col, perm, val, val_stride, x, y, vec_stride, part, pl.nslots, ind,
        lidx);
    if (pl.nfin > 0)
        plan_finish_kernel<T, IT>
            <<<dim3((pl.nfin + kWaves - 1) / kWaves, batch), kBlock, 0, s>>>(
                pl.fin, pl.nfin, part, pl.nslots, y, vec_stride, ind);
}

template <typename T, typename IT>
hipError_t launch_spmv(int slots, const IT *rp, const ColArgs &ca, const T *val,
                       int64_t val_stride, const T *x, T *y, int64_t n, int64_t vec_stride,
                       int batch, hipStream_t s, const RowPlan *plan,
                       const IterArgs<T, IT> *ind) {
    const dim3 grid(grid_for_tiles(tiles_of(n)), batch);
    const bool ps = planned(plan);
    const uint8_t *pt = ps ? plan->tiles : nullptr;
    if (!ps || !plan->all_tiles) {
        SLA_DISPATCH_CM(ca.mode, SLA_DISPATCH_SLOTS(slots, spmv_kernel<T, IT, kS, kC>
                                                    <<<grid, kBlock, 0, s>>>(rp, ca, val,
                                                                             val_stride, x, y, n,
                                                                             vec_stride, pt,
                                                                             ind)));
    }
    if (ps)
        launch_plan_spmv<T, IT, kPlanA>(*plan, rp, nullptr, val, val_stride, x, y, vec_stride,
                                        batch, s, ind);
    return hipGetLastError();
}

template <typename T, typename IT, bool GX, bool GV, bool NEG>
void launch_diag_vjp_t(const IT *rp, const ColArgs &ca, const T *val, int64_t val_stride,
                       const T *g, const T *x, T *gx, T *gv, int64_t n, int64_t nnz, int batch,
                       hipStream_t s) {
    const dim3 grid(grid_for_tiles(tiles_of(n)), batch);
    if (ca.nd <= 4)
        diag_vjp_kernel<T, IT, 4, GX, GV, NEG>
            <<<grid, kBlock, 0, s>>>(rp, ca, val, val_stride, g, x, gx, gv, n, nnz);
    else if (ca.nd <= 8)
        diag_vjp_kernel<T, IT, 8, GX, GV, NEG>
            <<<grid, kBlock, 0, s>>>(rp, ca, val, val_stride, g, x, gx, gv, n, nnz);
    else
        diag_vjp_kernel<T, IT, kMaxDiags, GX, GV, NEG>
            <<<grid, kBlock, 0, s>>>(rp, ca, val, val_stride, g, x, gx, gv, n, nnz);
}

template <typename T, typename IT>
hipError_t launch_diag_vjp(const IT *rp, const ColArgs &ca, const T *val, int64_t val_stride,
                           const T *g, const T *x, T *gx, T *gv, int64_t n, int64_t nnz,
                           int batch, bool neg, hipStream_t s) {
    if (gx && gv && !neg) {  // the product's backward: one pass
        launch_diag_vjp_t<T, IT, true, true, false>(rp, ca, val, val_stride, g, x, gx, gv, n, nnz,
                                                    batch, s);
        return hipGetLastError();
    }
    if (gx)
        launch_diag_vjp_t<T, IT, true, false, false>(rp, ca, val, val_stride, g, x, gx, gv, n,
                                                     nnz, batch, s);
    if (gv && neg)
        launch_diag_vjp_t<T, IT, false, true, true>(rp, ca, val, val_stride, g, x, gx, gv, n, nnz,
                                                    batch, s);
    else if (gv)
        launch_diag_vjp_t<T, IT, false, true, false>(rp, ca, val, val_stride, g, x, gx, gv, n,
                                                     nnz, batch, s);
    return hipGetLastError();
}

template <typename T, typename IT, bool NEG, bool GV, bool SC>
void launch_grad_t(const IT *rp, const ColArgs &ca, const T *g, const T *x, T *grad,
                   const T *val, const int32_t *pinv, T *c, int64_t n, int64_t nnz, int batch,
                   hipStream_t s, const RowPlan *plan) {
    const dim3 grid(grid_for_tiles(tiles_of(n)), batch);
    const bool ps = planned(plan);
    const uint8_t *pt = ps ? plan->tiles : nullptr;
    if (ps && plan->all_tiles) {
        // every tile is the plan's
    } else if (ca.mode == kColTile16) {
        grad_kernel<T, IT, NEG, kColTile16, GV, SC>
            <<<grid, kBlock, 0, s>>>(rp, ca, g, x, grad, val, pinv, c, n, nnz, pt);
    } else {
        grad_kernel<T, IT, NEG, kColWide, GV, SC>
            <<<grid, kBlock, 0, s>>>(rp, ca, g, x, grad, val, pinv, c, n, nnz, pt);
    }
    if (ps)
        plan_grad_kernel<T, IT, NEG, GV, SC>
            <<<dim3((plan->nitems + kNumXcd - 1) / kNumXcd * kNumXcd, batch), kBlock, 0, s>>>(
                plan->items, rp, plan->col, g, x, grad, val, pinv, c, n, nnz, plan->nitems);
}

template <typename T, typename IT>
hipError_t launch_grad(const IT *rp, const ColArgs &ca, const T *lam, const T *x, T *grad,
                       int64_t n, int64_t nnz, int batch, bool neg, hipStream_t s,
                       const RowPlan *plan) {
    if (ca.mode == kColDiag)
        return launch_diag_vjp<T, IT>(rp, ca, nullptr, 0, lam, x, nullptr, grad, n, nnz, batch,
                                      neg, s);
    if (neg)
        launch_grad_t<T, IT, true, true, false>(rp, ca, lam, x, grad, nullptr, nullptr, nullptr,
                                                n, nnz, batch, s, plan);
    else
        launch_grad_t<T, IT, false, true, false>(rp, ca, lam, x, grad, nullptr, nullptr, nullptr,
                                                 n, nnz, batch, s, plan);
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_terms_t(const IT *rp, const ColArgs &ca, const T *g, const T *val,
                          const int32_t *pinv, T *c, int64_t n, int64_t nnz, int batch,
                          hipStream_t s, const RowPlan *plan) {
    launch_grad_t<T, IT, false, false, true>(rp, ca, g, nullptr, nullptr, val, pinv, c, n, nnz,
                                             batch, s, plan);
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_rowsum(const IT *rp, const T *t, int64_t t_stride, const int32_t *perm,
                         const int32_t *col, const T *g, T *y, int64_t n, int batch,
                         hipStream_t s, const RowPlan *plan, const uint16_t *lidx) {
    const bool ps = planned(plan);
    const dim3 grid(grid_for_tiles(tiles_of(n)), batch);
    const uint8_t *pt = ps ? plan->tiles : nullptr;
    if (!ps || !plan->all_tiles) {
        if (perm)
            rowsum_kernel<T, IT, true><<<grid, kBlock, 0, s>>>(rp, t, t_stride, perm, col, g, y,
                                                               n, pt, nullptr);
        else
            rowsum_kernel<T, IT, false><<<grid, kBlock, 0, s>>>(rp, t, t_stride, nullptr,
                                                                nullptr, nullptr, y, n, pt, lidx);
    }
    if (ps) {
        if (perm)
            launch_plan_spmv<T, IT, kPlanPerm>(*plan, rp, perm, t, t_stride, g, y, n, batch, s);
        else
            launch_plan_spmv<T, IT, kPlanSum>(*plan, rp, nullptr, t, t_stride, nullptr, y, n,
                                              batch, s, nullptr, lidx);
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_scatter(const int32_t *pinv, const T *val, T *out, int64_t nnz,
                          hipStream_t s) {
    int64_t blocks = (nnz + kBlock - 1) / kBlock;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    scatter_kernel<T><<<(unsigned)blocks, kBlock, 0, s>>>(pinv, val, out, nnz);
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_dia_pack(const IT *rp, const ColArgs &cols, const T *val, int64_t val_stride,
                           T *out, int64_t n, int nsys, SolveState *st, hipStream_t s) {
    int64_t blocks = (n + kBlock - 1) / kBlock;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    dia_pack_kernel<T, IT><<<dim3((unsigned)blocks, nsys), kBlock, 0, s>>>(
        rp, cols, val, val_stride, out, n, cols.sym ? st : nullptr);
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

hipError_t launch_publish(const int32_t *ndone, int32_t *poll, hipStream_t s) {
    publish_kernel<<<1, 64, 0, s>>>(ndone, poll);
    return hipGetLastError();
}

#define SLA_INST(T, IT)                                                                         \
    template hipError_t launch_spmv<T, IT>(int, const IT *, const ColArgs &, const T *, int64_t, \
                                           const T *, T *, int64_t, int64_t, int, hipStream_t,   \
                                           const RowPlan *, const IterArgs<T, IT> *);           \
    template hipError_t launch_diag_vjp<T, IT>(const IT *, const ColArgs &, const T *, int64_t,  \
                                               const T *, const T *, T *, T *, int64_t, int64_t, \
                                               int, bool, hipStream_t);                          \
    template hipError_t launch_grad<T, IT>(const IT *, const ColArgs &, const T *, const T *,   \
                                           T *, int64_t, int64_t, int, bool, hipStream_t,       \
                                           const RowPlan *);                                    \
    template hipError_t launch_terms_t<T, IT>(const IT *, const ColArgs &, const T *,           \
                                              const T *, const int32_t *, T *, int64_t, int64_t, \
                                              int, hipStream_t, const RowPlan *);                \
    template hipError_t launch_rowsum<T, IT>(const IT *, const T *, int64_t, const int32_t *,  \
                                             const int32_t *, const T *, T *, int64_t, int,      \
                                             hipStream_t, const RowPlan *, const uint16_t *);    \
    template hipError_t launch_dinv<T, IT>(const IT *, const T *, int64_t, T *, int64_t,        \
                                           SolveState *, int, hipStream_t);                      \
    template hipError_t launch_dia_pack<T, IT>(const IT *, const ColArgs &, const T *, int64_t, \
                                               T *, int64_t, int, SolveState *, hipStream_t);

SLA_INST(float, int32_t)
SLA_INST(float, int64_t)
SLA_INST(double, int32_t)
SLA_INST(double, int64_t)
template hipError_t launch_scatter<float>(const int32_t *, const float *, float *, int64_t,
                                         hipStream_t);
template hipError_t launch_scatter<double>(const int32_t *, const double *, double *, int64_t,
                                          hipStream_t);
template hipError_t launch_zero_if<float>(const SolveState *, float *, int64_t, int, hipStream_t);
template hipError_t launch_zero_if<double>(const SolveState *, double *, int64_t, int,
                                           hipStream_t);

}  // namespace sla
