// Internal declarations of the gfx950 sparse-solve library.
//
// Layout in HBM: values [batch][nnz] (caller's, CSR order), vectors
// [batch][n]; every grid kernel walks rows in tiles of kTileRows and maps
// tiles to XCDs in contiguous ranges so that one XCD's L2 sees one slab of
// the matrix and the neighbouring vector entries it gathers.
#pragma once

#include <algorithm>
#include <cstddef>

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sla.h"

namespace sla {

#ifndef SLA_BLOCK
#define SLA_BLOCK 256
#endif
#ifndef SLA_BLOCKS_PER_XCD
#define SLA_BLOCKS_PER_XCD 128
#endif
constexpr int kBlock = SLA_BLOCK;  // threads per block of the grid kernels
constexpr int kWaveSize = 64;  // lanes of a wavefront
constexpr int kWaves = kBlock / kWaveSize;
constexpr int kTileRows = kBlock;  // rows per tile (one row per thread in
                                   // element-wise kernels)
constexpr int kNumXcd = 8;         // MI355X: 8 XCDs, 32 CUs each
// Grid kernels are persistent-style (a bounded grid strides over tiles):
// the number of blocks is also the number of partial sums that every block
// of the next kernel adds up, so it is kept moderate.
constexpr int kMaxBlocksPerXcd = SLA_BLOCKS_PER_XCD;
constexpr int kMaxGrid = kNumXcd * kMaxBlocksPerXcd;
constexpr int kMaxRed = 8;         // partial-sum slots
constexpr int kPartStride = kMaxRed * kMaxGrid;  // partial-sum doubles per system
constexpr int kBlockSolveThreads = 1024;
constexpr int kBlockSolveMaxN = 4096;  // 4 rows per thread; p, x, r, M^-1 in LDS

// Per-system solver state, device resident.  A field is written by block 0
// of one kernel and read by later kernels; fields that a kernel both reads
// and writes live in two slots selected by iteration parity, and the
// iteration counter is kept once per kernel role (iter_a read by the first
// kernel of an iteration, iter_b by the second).
struct SolveState {
    double rho[2];    // CG: gamma = r.u ; BiCGStab: rhat.r, by iteration parity
    double alpha[2];  // alpha by iteration parity
    double bb;        // ||rhs||^2
    double rr;        // ||r||^2 at the stop
    double half_ss;   // BiCGStab ||s||^2 of a half-step exit
    int32_t iter_a, iter_b;  // BiCGStab kernels
    int32_t iter_p[2];  // CG: iteration of the launch with parity 0 / 1
    int32_t iter;     // completed iterations at the stop
    int32_t done;     // 1 once converged / stopped (relaxed atomic access)
    int32_t status;   // sla_status of the system
    int32_t spmv;     // products with the operator
    int32_t nfused;   // launches of the fused SpMV kernels that did work
    int32_t zero_diag;
    int32_t zero_x;   // rhs == 0 with a user initial guess: x must become 0
    int32_t half_exit;  // BiCGStab: x took its half step, stop next kernel
    int32_t lag;      // CG: stopped at an odd iteration i with x = x_{i-1};
                      // the finishing launch adds alpha[0] p
    int32_t asym;     // diagonal-major pack: the values are not symmetric
};

// Sets *flag when any lane of the wavefront saw `bad`: one atomic per
// wavefront at most, none once the flag reads set (a check that fails
// everywhere would otherwise queue an atomic from every wavefront on one
// word).
__device__ __forceinline__ void raise_flag(int bad, int32_t *flag) {
    if (__any(bad) && (threadIdx.x & 63) == 0 &&
        __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0)
        atomicOr(flag, 1);
}

// Slots of the per-block partial sums ([kMaxRed][kMaxGrid] doubles).  A
// kernel reads only slots that the previous kernel wrote and writes only
// slots that it does not read.
enum : int {
    kCgGA = 0, kCgGA1 = 1, kCgDE = 2, kCgDE1 = 3, kCgRR = 4, kCgRR1 = 5, kCgBB = 6,
    kBiRV = 0, kBiTS = 1, kBiTT = 2, kBiSS = 3, kBiRS = 4, kBiRT = 5, kBiBB = 6, kBiRR = 7,
    kBiRR0 = 1,  // ||r_0||^2 of the init kernel, read by the first bicg_xpv only
};

// Device-resident arguments of the iteration kernels.  Kernels take a pointer
// to this block, so a captured HIP graph stays valid across calls while the
// host rewrites the pointers before each solve.
// Column modes of a pattern (how the SpMV-shaped kernels find the columns):
// the caller's int32 array, an int16 tile-relative copy, or per-row masks
// over at most kMaxDiags diagonals.  The solver iterations have one more
// form, kColDiaMajor: the values of the system repacked diagonal-major
// ([nd][n], zero where a row lacks a diagonal) for patterns on 3, 5 or 7
// diagonals (1D, 2D and 3D nearest-neighbour stencils), so that a row's
// entries need neither row pointers nor columns.
constexpr int kColWide = 0, kColTile16 = 1, kColDiag = 2, kColDiaMajor = 3;
constexpr int kMaxDiags = 16;
constexpr int kMaxDiaMajor = 8;  // diagonals a diagonal-major operator may have

struct ColArgs {
    const int32_t *col = nullptr;    // int32 columns (always present)
    const int16_t *col16 = nullptr;  // tile-relative int16 columns, or null
    const uint16_t *msk = nullptr;   // per-row diagonal masks, or null
    const int32_t *dlt = nullptr;    // [kMaxDiags] diagonal offsets, ascending (device)
    int32_t nneg = 0;                // diagonals below the main one
    int32_t mode = kColWide;
    int32_t nd = 0;                  // number of diagonals (kColDiag, kColDiaMajor)
    int32_t off[kMaxDiaMajor] = {};  // their offsets when nd <= kMaxDiaMajor
    // kColDiaMajor, CG only: the offsets mirror (off[q] = -off[nd-1-q]), so
    // when the system's values are symmetric (the pack found no pair
    // A[i][j], A[j][i] that differs in any bit) the iterations may read a
    // row's entries below the main diagonal from the upper diagonals of the
    // rows they mirror: A[i][i-d] = A[i-d][i]
    int32_t sym = 0;
    // kColDiaMajor, seven diagonals (0, +-1, +-N, +-D), CG: the plan of the
    // z-walk (cg_zwalk_plan) -- each plane of D rows cut into zw_ncol
    // columns of at most zw_tw rows, each column's zw_nz planes into zw_nseg
    // segments, one workgroup per segment; 0 when there is no z-walk
    int32_t zw_tw = 0, zw_ncol = 0, zw_nseg = 0, zw_nz = 0;
};

// Arguments of the grid iteration kernels for one system.  A launch that
// advances nsys systems of a batch at once reads an array of nsys of them,
// each already pointing at its system's data; workgroup (x, y) uses entry y.
template <typename T, typename IT>
struct IterArgs {
    const T *val;
    const IT *rp;
    ColArgs cols;
    T *x;
    const T *b;
    const T *dinv;
    T *r, *z, *q, *rh, *s, *t;
    T *p[2];
    T *v[2];
    SolveState *st;
    double *part;   // [kMaxRed][kMaxGrid]
    int32_t *ndone; // stopped systems of the launch (shared; the host waits for all)
    int64_t n;
    double tol;
    int32_t maxit;
    int32_t use_x0;
};

// Records a HIP error for sla_last_error (per calling thread).
void set_last_error(hipError_t e);

// ---------------------------------------------------------------- helpers

// v plus the value that the DPP move CTRL brings to this lane (both 32-bit
// halves moved in the VALU, no LDS traffic).  The row-local permutations
// write every lane; the row broadcasts leave the lanes of the first row(s)
// unwritten, whose results wave_sum does not read.  So the move needs no old
// value (giving it one, as update_dpp does, costs a zeroing move per half and
// step).
template <int CTRL>
__device__ __forceinline__ double dpp_add(double v) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(v);
    const int lo = __builtin_amdgcn_mov_dpp((int)(unsigned)u, CTRL, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_mov_dpp((int)(unsigned)(u >> 32), CTRL, 0xf, 0xf, false);
    return v + __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) |
                                                (unsigned)lo));
}

// Sum over each row of 16 lanes: pairs (quad_perm 1,0,3,2), quads (quad_perm
// 2,3,0,1), half rows (row_half_mirror), rows (row_mirror).  Each step adds
// two partial sums, in either order, so every lane of a row ends with the
// same bits.
__device__ __forceinline__ double row16_sum(double v) {
    v = dpp_add<0xB1>(v);
    v = dpp_add<0x4E>(v);
    v = dpp_add<0x141>(v);
    v = dpp_add<0x140>(v);
    return v;
}

__device__ __forceinline__ double lane_value(double v, int lane) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane((int)(unsigned)u, lane);
    const int hi = __builtin_amdgcn_readlane((int)(unsigned)(u >> 32), lane);
    return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) |
                                            (unsigned)lo));
}

// Sum over the wavefront as a uniform value: row sums r0..r3 by DPP, then
// row 3 adds row 2 and row 1 adds row 0 (row_bcast:15), row 3 adds row 1's
// total (row_bcast:31), and lane 63, (r3 + r2) + (r1 + r0), is read.  IEEE
// addition is commutative, so this is bitwise the sum (r0 + r1) + (r2 + r3)
// of the four row sums read one by one, in two DPP steps and two lane reads
// instead of eight lane reads, two moves and three adds.
__device__ __forceinline__ double wave_sum(double v) {
    v = row16_sum(v);
    v = dpp_add<0x142>(v);  // row_bcast:15
    v = dpp_add<0x143>(v);  // row_bcast:31
    return lane_value(v, 63);
}

// Contiguous tile range of this block's XCD, strided over the XCD's blocks.
// Requires gridDim.x to be a multiple of kNumXcd.
struct TileRange {
    int64_t first, end, stride;
};

constexpr int64_t kRoundsFrom = 16;  // tiles per block from which tiles go in rounds

__device__ __forceinline__ TileRange xcd_tiles(int64_t ntiles) {
    const int b = blockIdx.x;
    const int xcd = b % kNumXcd;
    const int local = b / kNumXcd;
    const int per = gridDim.x / kNumXcd;
    const int64_t chunk = (ntiles + kNumXcd - 1) / kNumXcd;
    const int64_t lo = (int64_t)xcd * chunk;
    int64_t hi = lo + chunk;
    if (hi > ntiles) hi = ntiles;
    TileRange tr;
    if (ntiles >= kRoundsFrom * (int64_t)gridDim.x) {
        // large systems: rounds of gridDim.x consecutive tiles, XCD x taking
        // the x-th run of `per` in each round, so the whole chip works on one
        // window of rows at a time and neighbours one grid plane away (3D
        // stencils) are still in the Infinity Cache when gathered
        tr.first = (int64_t)xcd * per + local;
        tr.end = ntiles;
        tr.stride = gridDim.x;
    } else {
        // one contiguous slab per XCD: its L2 holds the slab's neighbours
        tr.first = lo + local;
        tr.end = hi;
        tr.stride = per;
    }
    return tr;
}

// Block sums of NR per-thread values, stored by thread 0 in
// part[slot[r]][blockIdx.x] with plain stores: the kernel boundary publishes
// them to the next kernel.
template <int NR>
__device__ __forceinline__ void store_partials(double (&v)[NR], double *part, const int (&slot)[NR]) {
    __shared__ double red[NR][kWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const double w = wave_sum(v[r]);
        if (lane == 0) red[r][wave] = w;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            double s = 0.0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) s += red[r][w];
            part[slot[r] * kMaxGrid + blockIdx.x] = s;
        }
    }
}

// Totals of the partial sums a previous kernel of nb blocks stored; every
// block adds them in the same fixed order, so all blocks (and all runs) get
// bitwise the same totals.
template <int NR>
__device__ __forceinline__ void load_totals(const double *part, int nb, const int (&slot)[NR],
                                            double (&tot)[NR]) {
    __shared__ double red[NR][kWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        double s = 0.0;
        for (int j = threadIdx.x; j < nb; j += kBlock) s += part[slot[r] * kMaxGrid + j];
        s = wave_sum(s);
        if (lane == 0) red[r][wave] = s;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        double acc = 0.0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) acc += red[r][w];
        tot[r] = acc;
    }
    __syncthreads();
}

__device__ __forceinline__ int load_done(const SolveState *st) {
    return __hip_atomic_load(&st->done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Entry test of the iteration kernels.  Block 0 of the same launch may set
// `done` while this block's wavefronts are still starting, so wavefronts can
// read it differently; one that left at once would leave its share of the
// block's partial sums unwritten and the others would go on with a wrong
// total.  So each wavefront reads the flag once, records what it saw in
// seen[wave] and, if it saw the stop, skips its loads; the block acts on the
// records after its first barrier (any_saw_stop), every thread alike.
__device__ __forceinline__ bool saw_stop(const SolveState *st, int *seen) {
    const int d = __builtin_amdgcn_readfirstlane(load_done(st));
    if ((threadIdx.x & 63) == 0) seen[threadIdx.x >> 6] = d;
    return d != 0;
}
__device__ __forceinline__ bool any_saw_stop(const int *seen) {
    int a = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) a |= seen[w];
    return a != 0;
}
// The tiles a block walks, none for a wavefront that saw the stop.
__device__ __forceinline__ TileRange walk_tiles(int64_t ntiles, bool stopped) {
    TileRange tr = xcd_tiles(ntiles);
    if (stopped) tr.end = tr.first;
    return tr;
}

__device__ __forceinline__ bool block0() { return blockIdx.x == 0 && threadIdx.x == 0; }

// Block 0 of the system records the end of its solve and counts it in *ndone.
__device__ __forceinline__ void finish(SolveState *st, int32_t *ndone, int status, int iter,
                                       double rr) {
    if (block0()) {
        st->status = status;
        st->iter = iter;
        st->rr = rr;
        __hip_atomic_store(&st->done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(ndone, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Grid size for a tile count: a multiple of kNumXcd, at most kMaxGrid.
inline int grid_for_tiles(int64_t ntiles) {
    int64_t per = (ntiles + kNumXcd - 1) / kNumXcd;
    if (per > kMaxBlocksPerXcd) per = kMaxBlocksPerXcd;
    if (per < 1) per = 1;
    return (int)(per * kNumXcd);
}

__host__ __device__ inline int64_t tiles_of(int64_t n) { return (n + kTileRows - 1) / kTileRows; }

// Grid of a solve's fused kernels (init and iterations, which read each
// other's per-block partial sums, so they share it).  The diagonal-major
// tiles (cm == kColDiaMajor without the z-walk) run 96 workgroups per XCD
// at three waves per SIMD, which lets the compiler keep more of a row's
// loads in flight: on MI355X, CG on the 1e6-row 3D diffusion system 23.46
// -> 22.69 us per launch, BiCGStab on the 1024^2 upwind system 21.0 -> 20.5
// us.  The z-walk's plan and the other forms use grid_for_tiles.
constexpr int kDiaBlocksPerXcd = 96;
inline int iter_grid(int cm, int zw, int64_t n) {
    const int g = grid_for_tiles(tiles_of(n));
    return cm == kColDiaMajor && zw == 0 ? std::min(g, kNumXcd * kDiaBlocksPerXcd) : g;
}

// Tiles of the diagonal-major iteration kernels (not the z-walk), by
// dia_tile: kDiaTileGeneral, the general ones; kDiaTileFast, 32-bit byte
// offsets and the gathers of the -1 and +1 diagonals from the adjacent lanes
// (dia_rows ADJ), when every byte offset formed (at most nd * n values)
// fits 32 bits and the diagonals next to the main one are at -1 and +1;
// kDiaTilePair, the same with two rows per lane (dia_rows_pair), for fp64
// with n and every other offset even, on systems of more tiles than the
// grid's workgroups (below that, pairs would halve the grid rather than a
// workgroup's loads per row).
constexpr int kDiaTileGeneral = 0, kDiaTileFast = 1, kDiaTilePair = 2;
inline int dia_tile(const ColArgs &c, int64_t n, int64_t value_bytes) {
    if (c.mode != kColDiaMajor || c.nd < 3 || c.nd > kMaxDiaMajor) return kDiaTileGeneral;
    const int d0 = c.nd / 2;
    if ((int64_t)c.nd * n * value_bytes > (int64_t)0xffffffff || c.off[d0 - 1] != -1 ||
        c.off[d0 + 1] != 1)
        return kDiaTileGeneral;
    bool even = value_bytes == 8 && n % 2 == 0 && tiles_of(n) > kNumXcd * kDiaBlocksPerXcd;
    for (int q = 0; q < c.nd; ++q)
        if (q != d0 - 1 && q != d0 + 1) even = even && c.off[q] % 2 == 0;
    return even ? kDiaTilePair : kDiaTileFast;
}
// tiles of 2 * kTileRows rows (dia_rows_pair)
__host__ __device__ inline int64_t pair_tiles_of(int64_t n) {
    return (n + 2 * kTileRows - 1) / (2 * kTileRows);
}

// Gather slots per row for the row-per-lane SpMV from the longest row:
// 4, 6 or 8 (longer rows finish with a loop).
inline int slots_for(int64_t max_len) { return max_len <= 4 ? 4 : (max_len <= 6 ? 6 : 8); }

// ---------------------------------------------------------------- launchers
// (defined in the .hip files; all return hipError_t of the launch)

// Launch `k`; with `ev` (two events) the runtime records ev[0] when the
// kernel starts and ev[1] when it ends (hipExtLaunchKernel), so the pair
// times the kernel alone.  The iteration launchers take `ev` for the
// library's profile mode.
template <typename... KArgs, typename... Args>
inline void launch_maybe_timed(void (*k)(KArgs...), dim3 grid, dim3 block, uint32_t lds,
                               hipStream_t s, const hipEvent_t *ev, Args... args) {
    if (ev)
        hipExtLaunchKernelGGL(k, grid, block, lds, s, ev[0], ev[1], 0, args...);
    else
        hipLaunchKernelGGL(k, grid, block, lds, s, args...);
}

// The `slots` argument of the SpMV-shaped launchers is slots_for(longest row);
// `col16` (or `c16` for the kernels that read the argument block) selects the
// compact tile-relative columns when the handle has them.
// ------------------------------------------------------ rows past the stage
//
// A 256-row tile whose entries exceed kCap does not fit the tile walker's
// LDS stage, and in a tile that fits, a row longer than the walker's slots
// is summed by one thread with one gather after another.  For the
// stand-alone products and the gradient such tiles are planned once at
// set-up (the CSR-Adaptive idea of Greathouse and Daga, SC14: row blocks
// sized to the LDS, long rows split over workgroups):
//  - a short block: up to 256 consecutive rows of at most kShortRow entries
//    each and at most kPlanCap entries in all; one workgroup loads the
//    block's run coalesced, stages the products in LDS and sums each row in
//    entry order;
//  - a long row (more than kShortRow entries): chunks of kPlanCap entries,
//    one workgroup each, a fixed-order workgroup sum; a row of several
//    chunks leaves one partial per chunk and a last pass adds them in order.
// The tile kernels skip the tiles flagged in `tiles` when a plan covers them.
constexpr int kEpt = 8;              // staged entries per thread (tile walker)
constexpr int kCap = kBlock * kEpt;  // staged entries per tile
constexpr int kShortRow = 64;
#ifndef SLA_PLAN_EPT
#define SLA_PLAN_EPT 8
#endif
constexpr int kPlanEpt = SLA_PLAN_EPT;
constexpr int kPlanCap = kBlock * kPlanEpt;  // entries per short block or chunk
struct PlanItem {
    int32_t r0, r1;  // rows [r0, r1) (a long row's chunk: r1 = r0 + 1)
    int32_t slot;    // a chunk of a split row: its partial's slot; else -1
    int32_t kind;    // 0 short block, 1 long-row chunk
    int64_t e0, e1;  // entries [e0, e1)
};
struct PlanFin {
    int32_t row, slot0, nch, pad;  // a split row: its partials [slot0, slot0 + nch)
};
struct RowPlan {
    const uint8_t *tiles = nullptr;  // [tiles] 1 where the plan covers the tile
    bool all_tiles = false;          // it covers every tile: no tile kernel at all
    const PlanItem *items = nullptr;
    int32_t nitems = 0;
    const PlanFin *fin = nullptr;
    int32_t nfin = 0;
    int32_t nslots = 0;     // partials per system
    const int32_t *col = nullptr;  // the pattern's int32 columns
    void *part = nullptr;   // [systems of a launch][nslots] partial sums
};

// y = A x (plan: the tiles past the stage, or null).  ind: null, or a
// solver's device argument blocks, one per system of the launch; system y
// then takes its values from ind[y].val (val and val_stride are unused) and
// its product is skipped once ind[y].st has stopped.  Reading them there
// keeps a captured graph of these launches valid for every call.
template <typename T, typename IT>
hipError_t launch_spmv(int slots, const IT *rp, const ColArgs &ca, const T *val,
                       int64_t val_stride, const T *x, T *y, int64_t n, int64_t vec_stride,
                       int batch, hipStream_t s, const RowPlan *plan = nullptr,
                       const IterArgs<T, IT> *ind = nullptr);
// Backward of y = A x through A's diagonal masks (ca.mode == kColDiag), from
// A's own rows: gx = A^T g (when gx is not null, values val_stride apart) and
// gv[k] = g_i x_j on the pattern (when gv is not null; -g_i x_j with neg),
// one pass when both are wanted; vectors n apart, gv nnz apart.
template <typename T, typename IT>
hipError_t launch_diag_vjp(const IT *rp, const ColArgs &ca, const T *val, int64_t val_stride,
                           const T *g, const T *x, T *gx, T *gv, int64_t n, int64_t nnz,
                           int batch, bool neg, hipStream_t s);
// the gradient on the pattern; columns from ca as the products read them
template <typename T, typename IT>
hipError_t launch_grad(const IT *rp, const ColArgs &ca, const T *lam, const T *x, T *grad,
                       int64_t n, int64_t nnz, int batch, bool neg, hipStream_t s,
                       const RowPlan *plan = nullptr);
// A^T g for the per-entry column forms, first pass over A's rows: c[pinv[k]]
// = val[k] g_i, the terms in A^T's entry order (pinv: A's entry -> A^T's, or
// the handle's bpos, which lists the terms of the tiles launch_rowsum
// stages in LDS in A's order); g n apart, val and c nnz apart.
template <typename T, typename IT>
hipError_t launch_terms_t(const IT *rp, const ColArgs &ca, const T *g, const T *val,
                          const int32_t *pinv, T *c, int64_t n, int64_t nnz, int batch,
                          hipStream_t s, const RowPlan *plan = nullptr);
// y = A^T g row by row of A^T (rp, plan: A^T's row pointers and row plan),
// every row's terms rounded and added in entry order: the terms the scatter
// pass left in t (perm null; t_stride apart; with lidx, the handle's map
// of the tiles whose terms the pass wrote at bpos, in A's order), or A's
// values t through the transpose map perm with A^T's columns col and g
// (values t_stride apart, g and y n apart).
template <typename T, typename IT>
hipError_t launch_rowsum(const IT *rp, const T *t, int64_t t_stride, const int32_t *perm,
                         const int32_t *col, const T *g, T *y, int64_t n, int batch,
                         hipStream_t s, const RowPlan *plan = nullptr,
                         const uint16_t *lidx = nullptr);
// out[pinv[k]] = val[k]: one system's values in A^T's entry order.
template <typename T>
hipError_t launch_scatter(const int32_t *pinv, const T *val, T *out, int64_t nnz,
                          hipStream_t s);
// Diagonal-major copy of the CSR values of nsys systems (val_stride apart):
// out[s][q * n + i] = the entry of row i on diagonal q (bit q of msk[i]), 0
// where the row lacks it.  With st (cols.sym set: mirrored offsets), the
// same pass compares every entry below the main diagonal with its mirror
// bit for bit and sets st[s].asym when a pair differs or one of the two is
// missing.
template <typename T, typename IT>
hipError_t launch_dia_pack(const IT *rp, const ColArgs &cols, const T *val, int64_t val_stride,
                           T *out, int64_t n, int nsys, SolveState *st, hipStream_t s);
// per system of nsys: dinv[s][i] = 1 / val[s][diagpos[i]] (values val_stride apart)
template <typename T, typename IT>
hipError_t launch_dinv(const IT *diagpos, const T *val, int64_t val_stride, T *dinv, int64_t n,
                       SolveState *st, int nsys, hipStream_t s);

// CG (grid path, nsys systems per launch): init, then one launch per
// iteration with the iteration's parity
template <typename T, typename IT>
hipError_t launch_cg_init(int slots, int cm, int zw, bool jac, const IterArgs<T, IT> *a, int64_t n,
                          int nsys, hipStream_t s);
// zw: 0, or the z-walk (cg_zwalk_plan) with plain (1) or non-temporal (2)
// streams of the values and the vectors touched once; tile: dia_tile of the
// operator form (used without the z-walk)
template <typename T, typename IT>
hipError_t launch_cg_iter(int slots, int cm, bool jac, int zw, int tile,
                          const IterArgs<T, IT> *a, int64_t n, int nsys, int ph, hipStream_t s,
                          const hipEvent_t *ev = nullptr);
// The z-walk of a seven-diagonal operator form on n rows (3D stencils: a
// plane of D = off[6] rows, nz = n / D planes): fills it's zw_* fields and
// returns 1 (working set within the Infinity Cache: plain accesses) or 2
// (beyond it: non-temporal streams), or 0 when the walk does not apply
// (other forms, fewer than kZwMinPlanes planes per workgroup).
int cg_zwalk_plan(ColArgs &it, int64_t n, int64_t value_bytes);
// CG in three launches per iteration for operators with a row plan: init's
// first half (u_0, x), then per iteration the row updates (split_u), the
// product u -> v[0] through the plan (launch_spmv), and split_w (w^ and the
// partial sums; init = true after init's product)
template <typename T, typename IT>
hipError_t launch_cg_split_init(bool jac, const IterArgs<T, IT> *a, int64_t n, int nsys,
                                hipStream_t s);
template <typename T, typename IT>
hipError_t launch_cg_split_u(bool jac, const IterArgs<T, IT> *a, int64_t n, int nsys, int ph,
                             hipStream_t s);
template <typename T, typename IT>
hipError_t launch_cg_split_w(bool jac, bool init, const IterArgs<T, IT> *a, const IT *diagpos,
                             int64_t n, int nsys, int ph, hipStream_t s);

// BiCGStab (grid path; nsys systems, argument blocks a[0 .. nsys))
template <typename T, typename IT>
hipError_t launch_bicg_init(int cm, const IterArgs<T, IT> *a, int64_t n, int nsys, hipStream_t s);
// tile: dia_tile of the operator form
template <typename T, typename IT>
hipError_t launch_bicg_xpv(int slots, int cm, int tile, const IterArgs<T, IT> *a, int64_t n,
                           int nsys, hipStream_t s, const hipEvent_t *ev = nullptr);
template <typename T, typename IT>
hipError_t launch_bicg_st(int slots, int cm, int tile, const IterArgs<T, IT> *a, int64_t n,
                          int nsys, hipStream_t s, const hipEvent_t *ev = nullptr);
// BiCGStab in six launches per iteration for operators with a row plan:
// part 0 (first half's updates), [p -> v product], 1 (its partials),
// 2 (second half's updates), [s -> t product], 3 (its partials)
template <typename T, typename IT>
hipError_t launch_bicg_split(int part, const IterArgs<T, IT> *a, int64_t n, int nsys,
                             hipStream_t s);

// *poll = *ndone, poll being the device address of pinned host memory
hipError_t launch_publish(const int32_t *ndone, int32_t *poll, hipStream_t s);
// shared by both grid solvers: x = 0 when the state asks for it (nsys systems)
template <typename T>
hipError_t launch_zero_if(const SolveState *st, T *x, int64_t n, int nsys, hipStream_t s);
// After a grid CG solve: x += alpha[0] p when the stop left x one step behind.
template <typename T>
hipError_t launch_cg_lag(const SolveState *st, const T *p, T *x, int64_t n, int nsys,
                         hipStream_t s);

// CG, one workgroup per system (n <= kBlockSolveMaxN)
struct BlockCgParams {
    const void *val;
    const void *rp;
    const int32_t *col;
    const void *diagpos;
    void *x;
    const void *b;
    SolveState *st;
    int64_t n, nnz;
    double tol;
    int32_t maxit;
    int32_t use_x0;
    int32_t jac;
};
template <typename T, typename IT>
hipError_t launch_block_cg(int max_len, const BlockCgParams &p, int batch, hipStream_t s);

// Lanczos vector kernels and the eigenvalue gradient (kernels_eig.hip)
template <typename T>
hipError_t launch_eig_dots(const T *V, int m, const T *w, int64_t n, double *part, double *out,
                           bool root, hipStream_t s);
template <typename T>
hipError_t launch_eig_update(T *w, const T *V, int m, const double *c, int64_t n, hipStream_t s);
template <typename T>
hipError_t launch_eig_scale(const T *w, T *out, const double *beta, double tiny, int64_t n,
                            hipStream_t s);
template <typename T>
hipError_t launch_eig_combine(T *X, const T *V, int m, int k, const double *S, int64_t n,
                              hipStream_t s);
template <typename T, typename IT>
hipError_t launch_eig_outer(const IT *rp, const int32_t *col, const T *X, int k, const T *g,
                            T *grad, int64_t n, hipStream_t s);

// pattern setup

// Temporaries of the set-up, carved from one allocation that sla_create
// makes and releases (setup_scratch_bytes / setup_scratch_carve): the row
// of every entry, the transpose sort's keys (two buffers) and values, its
// digit counts, and the scans' tile totals.
struct SetupScratch {
    int32_t *rowidx = nullptr;    // [nnz] row of every entry of A
    int32_t *keys[2] = {nullptr, nullptr};
    int32_t *vals = nullptr;
    int32_t *hist = nullptr;
    int32_t *tot = nullptr;
    int32_t *rowidx_t = nullptr;  // after setup_transpose: row of every entry of A^T
};
int64_t setup_scratch_bytes(int64_t nnz, bool rowidx, bool transpose);
void setup_scratch_carve(void *base, int64_t nnz, bool rowidx, bool transpose, SetupScratch *out);
// whether a pattern is checked entry by entry (a row longer than kShortRow)
bool setup_entrywise(int32_t max_len, int64_t nnz);

// *bad = 1 when row_ptr is not a valid CSR row pointer (synchronizes `s`)
template <typename IT>
hipError_t setup_check_rowptr(const IT *rp, int64_t n, int64_t nnz, int32_t *flag, int32_t *bad,
                              hipStream_t s);
// rowidx[k] = row of entry k (a valid row_ptr; tot: scan totals)
template <typename IT>
hipError_t setup_row_index(const IT *rp, int64_t n, int64_t nnz, int32_t *rowidx, int32_t *tot,
                           hipStream_t s);
// *bad = 1 for a column out of range or out of order or a missing diagonal;
// diagpos[i] = position of A_ii.  rowidx: null (per-row checks) or the row
// of every entry (entry by entry).  Synchronizes `s`.
template <typename IT>
hipError_t setup_check_cols(const IT *rp, const int32_t *col, int64_t n, int64_t nnz,
                            const int32_t *rowidx, IT *diagpos, int32_t *flag, int32_t *bad,
                            hipStream_t s);
template <typename IT>
hipError_t setup_max_row(const IT *rp, int64_t n, int32_t *scratch, int32_t *out, hipStream_t s);
// Diagonal masks: the distinct column offsets (col - row) of the pattern
// when there are at most kMaxDiags of them (*ndiag = their number, else 0;
// dlt ascending, host array), then msk[i] = the set of diagonals row i
// stores (synchronizes `s`).
template <typename IT>
hipError_t setup_diag(const IT *rp, const int32_t *col, int64_t n, int32_t *dev_table,
                      int32_t *scratch, int32_t *dlt, int32_t *ndiag, hipStream_t s);
template <typename IT>
hipError_t setup_diag_masks(const IT *rp, const int32_t *col, int64_t n, const int32_t *dlt_dev,
                            int32_t ndiag, uint16_t *msk, hipStream_t s);
// Compact columns: out[k] = col[k] - (first row of row(k)'s tile) as int16.
// With out == nullptr only checks; *fits = 1 when every entry fits
// (synchronizes `s`).  rowidx: null (per row) or the row of every entry.
template <typename IT>
hipError_t setup_col16(const IT *rp, const int32_t *col, int64_t n, int64_t nnz,
                       const int32_t *rowidx, int16_t *out, int32_t *scratch, int32_t *fits,
                       hipStream_t s);
// The single checks behind the set-up steps, for callers that keep their
// own flags: *flag is raised (row pointers not monotone or not ending at
// nnz; a column out of range or out of order, or no diagonal), *out is
// atomically maxed with the longest row; both must start at 0.  The column
// check walks each row in one thread (meant for rows of modest length) and
// writes diagpos.  Nothing is allocated or synchronized.
template <typename IT>
hipError_t launch_check_rowptr(const IT *rp, int64_t n, int64_t nnz, int32_t *flag,
                               hipStream_t s);
template <typename IT>
hipError_t launch_check_cols_rows(const IT *rp, const int32_t *col, int64_t n, IT *diagpos,
                                  int32_t *flag, hipStream_t s);
template <typename IT>
hipError_t launch_max_row(const IT *rp, int64_t n, int32_t *out, hipStream_t s);
// The transpose map of a valid pattern whose row index is in scr.rowidx:
// rp_t [n+1], col_t [nnz] (row of each A^T entry), perm [nnz] (A's position
// of each A^T entry) and pinv [nnz] (A^T's position of each A entry);
// scr.rowidx_t is left pointing at the row of every A^T entry.  Synchronizes
// `s`.
template <typename IT>
hipError_t setup_transpose(const IT *rp, const int32_t *col, int64_t n, int64_t nnz, IT *rp_t,
                           int32_t *col_t, int32_t *perm, int32_t *pinv, SetupScratch &scr,
                           hipStream_t s);
// Write positions of the two-pass A^T products from the transpose map:
// bpos [nnz] (where the terms pass stores entry k's term) and lidx [nnz]
// (for each of those places in a tile the row sums stage in LDS, the
// entry's offset in A^T's order inside its tile or row-plan block), given
// A^T's row plan (empty or not).  Does not synchronize.
template <typename IT>
hipError_t setup_buckets(const IT *rp_t, const int32_t *perm, const RowPlan &plan_t, int64_t n,
                         int64_t nnz, int32_t *bpos, uint16_t *lidx, hipStream_t s);

}  // namespace sla
