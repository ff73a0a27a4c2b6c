// The tile loop shared by every SpMV-shaped grid kernel.
//
// A tile is kTileRows consecutive rows.  Their entries form one contiguous run
// [rp[row0], rp[row0 + rows]) of the value and column arrays, so the block
// reads that run as consecutive elements (entry e by thread e mod kBlock,
// kEpt entries per thread) into LDS.  The loads are unconditional (indices
// past the run are clamped to its last entry) so the compiler issues all of
// them before the first use.  After a barrier thread t walks row t from LDS
// and gathers its k-th neighbour for k = 0..SLOTS-1 in lock step with the
// other lanes (slots past the row repeat its last entry and are left out of
// the sum).  For banded and stencil matrices neighbouring rows have
// neighbouring columns, so each gather instruction touches a few consecutive
// cache lines.  Each row's sum is formed in entry order, one explicit fused
// multiply-add per entry (as are the kernels' dot-product partials), so every
// storage form and code path rounds the same way whatever the compiler would
// contract on its own; rows longer than SLOTS finish with a plain loop; a tile
// with more than kCap entries (long rows) is processed one wavefront per row,
// lanes striding over the row.
//
// Pipelining: the next tile's row pointers are loaded while this tile is
// processed and parked in a second LDS buffer; a row's own vector entries
// (the row functor's inputs) are loaded together with the tile's values.
// The first tile's row pointers share their barrier with the kernel's own
// start-up loads (the `pre` hook), and `post` may stop the kernel there.
#pragma once

#include "sla_internal.h"

namespace sla {

template <typename T>
using gptr = __attribute__((address_space(1))) T *;

// Pointers read from the argument block are generic; every array the kernels
// touch lives in global memory, so say so and get global (not flat) accesses.
template <typename T>
__device__ __forceinline__ gptr<T> glb(T *p) {
    return (gptr<T>)p;
}

// &v[i] formed as v plus a 32-bit byte offset (O32), or as usual.  With O32
// a load or store takes v from scalar registers and one 32-bit offset
// register, which the three vectors gathered at one column share.  With
// 64-bit element addresses each of the thirty-odd memory accesses of a row
// holds a register pair, and the compiler, short of registers, waited for all
// loads in flight several times per tile (CG on the 1e6-row 3D diffusion
// system: 24.7 -> 23.4 us per launch).  Valid when every byte offset formed fits 32 bits.
template <bool O32, typename T>
__device__ __forceinline__ gptr<T> elem(gptr<T> v, int64_t i) {
    if constexpr (O32) {
        typedef __attribute__((address_space(1))) unsigned char byte_t;
        return (gptr<T>)((byte_t *)v + (uint32_t)i * (uint32_t)sizeof(T));
    } else {
        return v + i;
    }
}

__device__ __forceinline__ float wave_sum_t(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}
__device__ __forceinline__ double wave_sum_t(double v) { return wave_sum(v); }

struct NoPre {
    __device__ void operator()() const {}
};
struct NoPost {
    __device__ bool operator()() const { return true; }
};
struct NoOwn {
    __device__ int operator()(int64_t) const { return 0; }
};

// Loads the previous kernel's per-block partial sums of NR slots and leaves
// each wavefront's sum in red[r][wave]; totals() adds the wavefront sums in
// order after a barrier (all blocks get bitwise the same totals).
template <int NR>
__device__ __forceinline__ void partial_loads(const double *part, const int (&slot)[NR],
                                              double (*red)[kWaves]) {
    const gptr<const double> pg = glb(part);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    double a[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) a[r] = 0.0;
    for (int j = tid; j < (int)gridDim.x; j += kBlock) {
#pragma unroll
        for (int r = 0; r < NR; ++r) a[r] += pg[slot[r] * kMaxGrid + j];
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const double w = wave_sum(a[r]);
        if (lane == 0) red[r][wave] = w;
    }
}

template <int NR>
__device__ __forceinline__ void totals(double (*red)[kWaves], double (&tot)[NR]) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        double acc = 0.0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) acc += red[r][w];
        tot[r] = acc;
    }
}

// Loads gathered at one column, combined after all of a round are issued.
template <typename T>
struct G2 {
    T a, b;
};
template <typename T>
struct G3 {
    T a, b, c;
};
template <typename T>
struct G4 {
    T a, b, c, d;
};

// v[k] through the scalar data cache: k must be the same in every lane of
// the wavefront, and nothing may write v while the kernel runs (the cache is
// invalidated when a kernel starts, not when another one writes).
template <typename T>
__device__ __forceinline__ T sld(gptr<const T> v, int64_t k) {
    return ((const __attribute__((address_space(4))) T *)v)[k];
}

// Lane shifts of the wavefront by DPP: CTRL 0x138 (wave_shr:1) gives lane t
// the value of lane t - 1 and lane 0 `edge`; 0x130 (wave_shl:1) gives lane t
// the value of lane t + 1 and lane 63 `edge`.  A move, so the bits are kept.
template <int CTRL, typename T>
__device__ __forceinline__ T lane_shift(T v, T edge) {
    static_assert(CTRL == 0x138 || CTRL == 0x130, "wave_shr:1 or wave_shl:1");
    if constexpr (sizeof(T) == 8) {
        const uint64_t b = __builtin_bit_cast(uint64_t, v), e = __builtin_bit_cast(uint64_t, edge);
        const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)e, (int)(uint32_t)b,
                                                                  CTRL, 0xf, 0xf, false);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(
            (int)(uint32_t)(e >> 32), (int)(uint32_t)(b >> 32), CTRL, 0xf, 0xf, false);
        return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
    } else {
        static_assert(sizeof(T) == 4, "4- or 8-byte values");
        return __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, edge),
                                                                 __builtin_bit_cast(int, v), CTRL,
                                                                 0xf, 0xf, false));
    }
}
template <int CTRL, typename T>
__device__ __forceinline__ G2<T> lane_shift(const G2<T> &v, const G2<T> &e) {
    return G2<T>{lane_shift<CTRL>(v.a, e.a), lane_shift<CTRL>(v.b, e.b)};
}
template <int CTRL, typename T>
__device__ __forceinline__ G3<T> lane_shift(const G3<T> &v, const G3<T> &e) {
    return G3<T>{lane_shift<CTRL>(v.a, e.a), lane_shift<CTRL>(v.b, e.b), lane_shift<CTRL>(v.c, e.c)};
}
template <int CTRL, typename T>
__device__ __forceinline__ G4<T> lane_shift(const G4<T> &v, const G4<T> &e) {
    return G4<T>{lane_shift<CTRL>(v.a, e.a), lane_shift<CTRL>(v.b, e.b), lane_shift<CTRL>(v.c, e.c),
                 lane_shift<CTRL>(v.d, e.d)};
}

// Gathering one vector entry: the load and the use are the same.
struct PlainGather {
    template <typename V>
    __device__ V operator()(V v) const { return v; }
};

// Largest divisor of slots that does not exceed round (rounds must tile the
// slots exactly).
constexpr int round_for(int slots, int round) {
    int r = round < slots ? round : slots;
    while (slots % r) --r;
    return r;
}

// Where the kernels read column indices (CM, the column mode):
//   kColWide   the caller's int32 array;
//   kColTile16 a compact copy built at set-up when every entry fits, the
//              int16 offset of the column from the first row of the entry's
//              tile (col = tile row0 + offset): 2 bytes per entry;
//   kColDiag   for patterns whose entries lie on at most 16 diagonals (grid
//              stencils) and whose rows hold at most 8 entries: one 16-bit
//              mask per row says which diagonals the row stores; the column
//              of diagonal q is row + dlt[q] (dlt ascending, so the row's
//              columns ascend with q): 2 bytes per row, no per-entry index.
//   kColDiaMajor  (solver iterations) the values are a diagonal-major copy,
//              vf(q * n + i) is row i's entry on diagonal q (0 where the row
//              lacks it) and its column is i + off[q]: no index at all.
template <int CM>
struct ColSrc {
    gptr<const int32_t> c32;
    gptr<const int16_t> c16;
    gptr<const uint16_t> msk;
    gptr<const int32_t> dlt;
    int32_t nneg;  // diagonals below the main one (dlt[q] < 0 for q < nneg)
    int32_t off[kMaxDiaMajor];  // kColDiaMajor: the diagonals' offsets, ascending
    // kColDiaMajor: the values are symmetric and the offsets mirror, so row
    // i's entry on a diagonal q below the main one is read as the entry of
    // row i + off[q] on the mirrored diagonal (uniform across the grid)
    int32_t sym;
    int32_t zw_tw, zw_ncol, zw_nseg, zw_nz;  // the z-walk's plan (ColArgs)
    // column of stored entry k in the tile starting at row0 (per-entry modes)
    __device__ __forceinline__ int32_t operator()(int64_t k, int64_t row0) const {
        if constexpr (CM == kColTile16)
            return (int32_t)row0 + (int32_t)c16[k];
        else
            return c32[k];
    }
};
template <int CM>
__device__ __forceinline__ ColSrc<CM> col_src(const ColArgs &a) {
    ColSrc<CM> c{glb(a.col), glb(a.col16), glb(a.msk), glb(a.dlt), a.nneg, {}, 0, 0, 0, 0, 0};
    if constexpr (CM == kColDiaMajor) {
#pragma unroll
        for (int q = 0; q < kMaxDiaMajor; ++q) c.off[q] = a.off[q];
        c.sym = a.sym;
        c.zw_tw = a.zw_tw;
        c.zw_ncol = a.zw_ncol;
        c.zw_nseg = a.zw_nseg;
        c.zw_nz = a.zw_nz;
    }
    return c;
}

// Index of the s-th set bit of m (s < popcount(m)).
__device__ __forceinline__ int nth_bit(uint32_t m, int s) {
    for (int i = 0; i < s; ++i) m &= m - 1;
    return __builtin_ctz(m);
}

template <typename T, typename IT>
struct RowLds {
    IT rp[2][kTileRows + 1];
    T val[kCap];
    int32_t col[kCap];
    int32_t dtab[kMaxDiags];  // diagonal offsets (kColDiag)
};

// Row i's entry on diagonal q of a diagonal-major operator.  Below the main
// diagonal with col.sym: the entry of row j = i + off[q] on the mirrored
// diagonal ND - 1 - q, whose column is i (no such row above the first: 0).
// One load either way, its address chosen by selects, so that the loads of
// a tile still issue back to back.
template <typename T, int ND, typename VF>
__device__ __forceinline__ T dia_entry(VF vf, const ColSrc<kColDiaMajor> &col, int q, int64_t i,
                                       int64_t n) {
    const int64_t own = (int64_t)q * n + i;
    if (2 * q + 1 >= ND) return vf(own);
    const int64_t j = i + col.off[q];
    const bool mir = col.sym != 0;
    const T v = vf(mir && j >= 0 ? (int64_t)(ND - 1 - q) * n + j : own);
    return mir && j < 0 ? T(0) : v;
}

// Rows of a diagonal-major operator with ND diagonals, the main one in the
// middle (slot ND / 2; the spmv_rows contract below, without the LDS): thread
// t of a tile takes row row0 + t and reads its ND values as ND coalesced
// loads, vf(q * n + i); the column of slot q is i + off[q], clamped into
// [0, n) for the zero padding slots of boundary rows (0 * finite adds
// nothing, so the sum over q -- ascending columns, the order of the CSR
// forms -- equals the sum over the stored entries).  The main diagonal's
// gathers use the row index itself, so they coincide with the row's own
// loads.  With SYM and col.sym the slots below the main diagonal are read
// from the mirrored diagonal at row i + off[q] (0 above the first row): the
// same bits as the row's own copy, so the sums do not change, and the lower
// copies' bytes are not read (their lines are the upper diagonals' lines of
// rows just before, mostly still in the caches).  All loads of a tile are issued
// before its first use, and the first tile's before the start-up barrier,
// so that their latency overlaps the kernel's start-up loads.
//
// ADJ (the diagonals next to the main one are at -1 and +1): the gathers of
// those two diagonals are the main diagonal's gathers of the rows before and
// after, which the neighbouring lanes hold, so they move across by lane
// shifts instead of being loaded again; lane 0 and lane 63 take theirs from
// uniform loads through the scalar cache, gs(c) (and vs(k) for values).
// With SYM the -1 diagonal's mirrored value (row i - 1's entry on the +1
// diagonal) comes from lane t - 1 the same way.  The texture addresser's
// work per row falls by seven of thirty wavefront loads in the CG iteration;
// it bounded the kernel (busy for 60-66 % of its cycles on the 1e6-row 3D
// diffusion system).  The values moved are the bits the loads would return,
// so the sums are unchanged.  gf, gs and vs must read arrays that the
// kernel does not write.
template <typename T, int ND, bool SYM, bool ADJ = false, typename VF, typename GF, typename CF,
          typename OF, typename RF, typename PRE, typename POST, typename VS = std::nullptr_t,
          typename GS = std::nullptr_t>
__device__ __forceinline__ bool dia_rows(const TileRange &tr, int64_t n,
                                         const ColSrc<kColDiaMajor> &col, VF vf, GF gf, CF cf,
                                         OF of, RF rf, PRE pre, POST post, VS vs = nullptr,
                                         GS gs = nullptr) {
    static_assert(ND >= 1 && ND <= kMaxDiaMajor && (ND & 1), "diagonal count");
    static_assert(!ADJ || ND >= 3, "ADJ: diagonals on both sides of the main one");
    using G = decltype(gf(0));
    using O = decltype(of(0));
    constexpr int d0 = ND / 2;  // the main diagonal's slot
    const int tid = threadIdx.x;
    T v[ND];
    G g[ND];
    O own;
    G elo{}, ehi{};  // ADJ: the gathers of rows wb - 1 and wb + 64
    T ev = T(0);     // ADJ with SYM: row wb - 1's entry on the +1 diagonal
    // ADJ with SYM: the -1 diagonal's value comes from lane t - 1
    auto shifted_val = [&](int q) { return ADJ && SYM && q == d0 - 1 && col.sym != 0; };
    auto load = [&](int64_t t) {
        const int64_t row0 = t * kTileRows;
        const int64_t left = n - row0;
        const int64_t i = row0 + (tid < left ? tid : left - 1);
        own = of(i);
#pragma unroll
        for (int q = 0; q < ND; ++q) {
            if (!shifted_val(q)) {
                if constexpr (SYM)
                    v[q] = dia_entry<T, ND>(vf, col, q, i, n);
                else
                    v[q] = vf((int64_t)q * n + i);
            }
            if (ADJ && (q == d0 - 1 || q == d0 + 1)) continue;
            int64_t c = i + col.off[q];
            c = c < 0 ? 0 : (c >= n ? n - 1 : c);
            g[q] = gf(q == d0 ? (int32_t)i : (int32_t)c);
        }
        if constexpr (ADJ) {
            // lane 0's row wb (rows past n take row n - 1, as above); its
            // neighbours clamped into [0, n) like the gathered columns
            const int64_t wb = row0 + kWaveSize * (int64_t)__builtin_amdgcn_readfirstlane(tid >> 6);
            const int64_t lo = wb < 1 ? 0 : (wb - 1 < n ? wb - 1 : n - 1);
            const int64_t hi = wb + kWaveSize < n ? wb + kWaveSize : n - 1;
            elo = gs(lo);
            ehi = gs(hi);
            if constexpr (SYM) {
                if (col.sym) ev = wb >= 1 ? vs((int64_t)(d0 + 1) * n + lo) : T(0);
            }
        }
    };
    auto use = [&](int64_t t) {
        const int64_t i = t * kTileRows + tid;
        if constexpr (ADJ) {
            g[d0 - 1] = lane_shift<0x138>(g[d0], elo);
            g[d0 + 1] = lane_shift<0x130>(g[d0], ehi);
            if (shifted_val(d0 - 1)) v[d0 - 1] = lane_shift<0x138>(v[d0 + 1], ev);
        }
        T s = T(0);
#pragma unroll
        for (int q = 0; q < ND; ++q) s = fma(v[q], cf(g[q]), s);
        if (i < n) rf(i, s, own, v[d0]);
    };
    int64_t t = tr.first;
    if (t < tr.end) load(t);
    pre();
    __syncthreads();
    if (!post()) return false;
    if (t < tr.end) use(t);
    for (t += tr.stride; t < tr.end; t += tr.stride) {
        load(t);
        use(t);
    }
    return true;
}

// Two consecutive fp64 values, 8-byte aligned: one 16-byte wavefront load
// or store (global memory needs 4-byte alignment for it).
typedef double pair_t __attribute__((ext_vector_type(2), aligned(8)));

// Row H (0: the first, 1: the second) of a pair, for a gather of several
// vectors at one column.
template <int H>
__device__ __forceinline__ double half(pair_t v) {
    return H ? v.y : v.x;
}
template <int H>
__device__ __forceinline__ G2<double> half(const G2<pair_t> &v) {
    return G2<double>{half<H>(v.a), half<H>(v.b)};
}
template <int H>
__device__ __forceinline__ G3<double> half(const G3<pair_t> &v) {
    return G3<double>{half<H>(v.a), half<H>(v.b), half<H>(v.c)};
}
template <int H>
__device__ __forceinline__ G4<double> half(const G4<pair_t> &v) {
    return G4<double>{half<H>(v.a), half<H>(v.b), half<H>(v.c), half<H>(v.d)};
}

// dia_rows (with ADJ) for fp64 values taking two consecutive rows per lane:
// lane t of a tile of 2 * kTileRows rows takes rows i = row0 + 2t and i + 1,
// and every load and store moves the pair's two values as one 16-byte
// access.  On MI355X a wavefront load of 16 bytes per lane keeps the texture
// addresser busy about 20 cycles and one of 8 bytes about 18 (a probe of L2
// resident loads), so the pairs need little more than half of its time per
// row; CG on the 1e6-row 3D diffusion system: 21.6 -> 20.2 us per launch.
// Requires n even and every offset but the -1 and +1 ones even, so that no
// pair straddles the ends of a vector: the pair at an even column c holds
// columns c and c + 1, both inside [0, n) or both outside (those clamped to
// the pair at 0 or n - 2; their padding values are 0).  The -1 and +1
// gathers come from the lane's own pair and, for the rows at its ends, from
// lanes t - 1 and t + 1 by lane shifts (gs at a wavefront's edges); with SYM
// the -1 diagonal's values are row i - 1's (lane t - 1, or vs) and row i's
// entries on the +1 diagonal.  vf2, gf2 and of2 load pairs; rf2(i, s0, s1,
// own, d0, d1) consumes both rows' products and diagonal entries.  A row's
// terms and their order are those of dia_rows; each thread adds its two
// rows' contributions to the partial sums in row order, so the partial sums
// are added in another order than with one row per lane.
template <int ND, bool SYM, typename VF2, typename VS, typename GF2, typename GS, typename CF,
          typename OF2, typename RF2, typename PRE, typename POST>
__device__ __forceinline__ bool dia_rows_pair(const TileRange &tr, int64_t n,
                                              const ColSrc<kColDiaMajor> &col, VF2 vf2, VS vs,
                                              GF2 gf2, GS gs, CF cf, OF2 of2, RF2 rf2, PRE pre,
                                              POST post) {
    static_assert(ND >= 3 && ND <= kMaxDiaMajor && (ND & 1), "diagonal count");
    using GP = decltype(gf2(0));  // the gathered vectors' pairs at a column
    using G = decltype(gs(0));    // the same for one row
    using O = decltype(of2(0));
    constexpr int d0 = ND / 2;
    constexpr int64_t kRows = 2 * kTileRows;
    const int tid = threadIdx.x;
    const int64_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool msym = SYM && col.sym != 0;
    pair_t v[ND];
    GP g[ND];
    O own;
    G elo{}, ehi{};  // the gathers of rows wb - 1 and wb + 128
    double ev = 0.0;  // with msym: row wb - 1's entry on the +1 diagonal
    auto load = [&](int64_t t) {
        const int64_t row0 = t * kRows;
        int64_t i = row0 + 2 * tid;
        i = i < n - 2 ? i : n - 2;  // pairs past the end read the last one
        own = of2(i);
#pragma unroll
        for (int q = 0; q < ND; ++q) {
            if (q == d0 - 1 && msym) {
                // from lane t - 1 and this pair's +1 diagonal
            } else if (SYM && q < d0 && msym) {
                // rows i + off[q] and i + 1 + off[q] on the mirrored diagonal
                const int64_t j = i + col.off[q];
                const pair_t m = vf2(j >= 0 ? (int64_t)(ND - 1 - q) * n + j : (int64_t)q * n + i);
                v[q] = j >= 0 ? m : pair_t{0.0, 0.0};
            } else {
                v[q] = vf2((int64_t)q * n + i);
            }
            if (q == d0 - 1 || q == d0 + 1) continue;
            int64_t c = i + col.off[q];
            c = c < 0 ? 0 : (c > n - 2 ? n - 2 : c);
            g[q] = gf2(q == d0 ? i : c);
        }
        const int64_t wb = row0 + 2 * kWaveSize * wave;  // lane 0's first row
        const int64_t lo = wb < 1 ? 0 : (wb - 1 < n ? wb - 1 : n - 1);
        const int64_t hi = wb + 2 * kWaveSize < n ? wb + 2 * kWaveSize : n - 1;
        elo = gs(lo);
        ehi = gs(hi);
        if constexpr (SYM) {
            if (msym) ev = wb >= 1 ? vs((int64_t)(d0 + 1) * n + lo) : 0.0;
        }
    };
    auto use = [&](int64_t t) {
        const int64_t i = t * kRows + 2 * tid;
        const G g0 = half<0>(g[d0]), g1 = half<1>(g[d0]);
        const G gm = lane_shift<0x138>(g1, elo);  // row i - 1
        const G gp = lane_shift<0x130>(g0, ehi);  // row i + 2
        double m0, m1;  // the -1 diagonal's values of rows i and i + 1
        if (msym) {
            m0 = lane_shift<0x138>(v[d0 + 1].y, ev);
            m1 = v[d0 + 1].x;
        } else {
            m0 = v[d0 - 1].x;
            m1 = v[d0 - 1].y;
        }
        double s0 = 0.0, s1 = 0.0;
#pragma unroll
        for (int q = 0; q < ND; ++q) {
            if (q == d0 - 1) {
                s0 = fma(m0, cf(gm), s0);
                s1 = fma(m1, cf(g0), s1);
            } else if (q == d0) {
                s0 = fma(v[q].x, cf(g0), s0);
                s1 = fma(v[q].y, cf(g1), s1);
            } else if (q == d0 + 1) {
                s0 = fma(v[q].x, cf(g1), s0);
                s1 = fma(v[q].y, cf(gp), s1);
            } else {
                s0 = fma(v[q].x, cf(half<0>(g[q])), s0);
                s1 = fma(v[q].y, cf(half<1>(g[q])), s1);
            }
        }
        if (i < n) rf2(i, s0, s1, own, v[d0].x, v[d0].y);
    };
    int64_t t = tr.first;
    if (t < tr.end) load(t);
    pre();
    __syncthreads();
    if (!post()) return false;
    if (t < tr.end) use(t);
    for (t += tr.stride; t < tr.end; t += tr.stride) {
        load(t);
        use(t);
    }
    return true;
}

// Rows of a seven-diagonal operator walked along its outermost offset
// D = off[6] = -off[0] (a 3D stencil's plane of D rows; off[2] = -1,
// off[4] = 1).  The plan (cg_zwalk_plan, in col.zw_*) cuts every plane into
// zw_ncol columns of zw_tw consecutive rows (the last one possibly narrower)
// and the zw_nz planes of each column into zw_nseg segments; workgroup b
// takes one segment and walks it plane by plane, lane t taking in-plane row
// column * zw_tw + t, so its next rows are the plane above its current ones,
// lane for lane.  Segments are numbered column by column and each XCD takes
// a contiguous range of them, so a column's segments and its neighbouring
// columns (the +-N gathers) share an L2.  The block keeps, per lane, the
// gathered entries of its column in planes z - 1, z and z + 1 in an LDS
// ring: the +D gathers of plane z are plane z + 1's own entries, so a
// segment reads each plane's entries from memory once (plus the plane
// below its first one); the -D, own and (inside the column) +-1 gathers
// come from the ring, the +-N gathers and the column-edge +-1 from memory.
// ofz(i, g) builds a row's own inputs from its gathered entries g.  The
// terms and their order are those of dia_rows, so every row's sum is
// bitwise the same.  With col.sym the -D entry of a row is the +D entry of
// the row one plane below, which this lane loaded for its previous plane: it
// is carried in a register, and the -1 and -N entries are read from their
// mirrors as in dia_rows.  The values of the +-1 and +-N diagonals then go
// through vk (loads that keep their lines cached, since the mirrored reads
// come back to them), the others through vf.  With one segment per column
// and 256-row columns this is the assignment of the tiles in rounds
// (xcd_tiles), so the partial sums are also those of the other forms.
template <typename T, typename VF, typename VK, typename GF, typename CF, typename OF,
          typename RF, typename PRE, typename POST, typename G>
__device__ __forceinline__ bool dia_rows_zw(bool active, int64_t n,
                                            const ColSrc<kColDiaMajor> &col, VF vf, VK vk, GF gf,
                                            CF cf, OF ofz, RF rf, PRE pre, POST post,
                                            G (*ring)[kTileRows]) {
    constexpr int ND = 7, d0 = 3;
    const int tid = threadIdx.x;
    const int64_t D = col.off[6];
    // this workgroup's segment
    const int xcd = blockIdx.x % kNumXcd, local = blockIdx.x / kNumXcd;
    const int64_t total = (int64_t)col.zw_ncol * col.zw_nseg;
    const int64_t lo = total * xcd / kNumXcd, hi = total * (xcd + 1) / kNumXcd;
    const int64_t seg = lo + local;
    if (seg >= hi) active = false;
    const int64_t c = active ? seg / col.zw_nseg : 0;
    const int64_t sg = active ? seg % col.zw_nseg : 0;
    const int64_t z0 = active ? col.zw_nz * sg / col.zw_nseg : 0;
    const int64_t z1 = active ? col.zw_nz * (sg + 1) / col.zw_nseg : 0;
    const int64_t j0 = c * col.zw_tw;
    const int64_t wl = D - j0 < col.zw_tw ? D - j0 : col.zw_tw;  // lanes of this column
    const bool lane_on = tid < wl;
    const int64_t j = j0 + (lane_on ? tid : wl - 1);  // in-plane row (clamped)
    auto clampc = [&](int64_t x) -> int32_t {
        return (int32_t)(x < 0 ? 0 : (x >= n ? n - 1 : x));
    };
    int prev = 2, cur = 0, next = 1;
    T vd = T(0);  // col.sym: the previous plane's +D entry
    bool carried = false;
    if (z0 < z1) {
        // the plane below the first one: padding below the grid
        ring[prev][tid] = z0 > 0 ? gf((int32_t)((z0 - 1) * D + j)) : G{};
        ring[cur][tid] = gf((int32_t)(z0 * D + j));
    }
    pre();
    __syncthreads();
    if (!post()) return false;
    for (int64_t z = z0; z < z1; ++z) {
        const int64_t i = z * D + j;
        T v[ND];
        G g[ND];
#pragma unroll
        for (int q = 0; q < ND; ++q) {
            if (q == 0 && col.sym && carried)
                v[q] = vd;
            else if (col.sym && q != 0 && q != d0 && q != 6)
                v[q] = dia_entry<T, ND>(vk, col, q, i, n);
            else
                v[q] = dia_entry<T, ND>(vf, col, q, i, n);
        }
        vd = v[6];
        carried = true;
        g[6] = gf(clampc(i + col.off[6]));
        g[1] = gf(clampc(i + col.off[1]));
        g[5] = gf(clampc(i + col.off[5]));
        g[2] = tid > 0 ? ring[cur][tid - 1] : gf(clampc(i - 1));
        g[4] = tid < wl - 1 ? ring[cur][tid + 1] : gf(clampc(i + 1));
        g[0] = ring[prev][tid];
        g[3] = ring[cur][tid];
        const auto own = ofz(i, g[3]);
        ring[next][tid] = g[6];
        T s = T(0);
#pragma unroll
        for (int q = 0; q < ND; ++q) s = fma(v[q], cf(g[q]), s);
        if (lane_on) rf(i, s, own, v[d0]);
        // the next plane's ring slot is complete, and this plane's reads of
        // the slot about to be overwritten are done
        __syncthreads();
        const int o = prev;
        prev = cur;
        cur = next;
        next = o;
    }
    return true;
}

// col: the column source (per-entry columns, or per-row diagonal masks);
// vf(k): value of stored entry k; gf(c): the loads gathered at column c;
// cf(g): the vector entry those loads make (the gathers of ROUND slots are
// all issued before the first cf); of(i): this thread's own-row inputs,
// loaded early (i is clamped into the tile, so the load is always in bounds);
// rf(i, s, own, d): consumes row i's product s; d is the row's diagonal entry
// (the stored entry whose column is i; every validated pattern has one).
// pre(): start-up loads issued with the first row pointers (no barrier
// inside); post(): runs after the first barrier, every thread, and returns
// false to end the kernel (the same in every thread).  plan_tiles: when not
// null, the tiles it flags are left alone (a row plan covers them).  SYM:
// a diagonal-major operator honours col.sym (CG instantiations only).
template <typename T, typename IT, int SLOTS, int ROUND, int CM, bool SYM = false, typename VF,
          typename GF, typename CF, typename OF, typename RF, typename PRE, typename POST>
__device__ __forceinline__ bool spmv_rows(const TileRange &tr, int64_t n, gptr<const IT> rp,
                                          ColSrc<CM> col, RowLds<T, IT> &sm, VF vf, GF gf, CF cf,
                                          OF of, RF rf, PRE pre, POST post,
                                          const uint8_t *plan_tiles = nullptr) {
    if constexpr (CM == kColDiaMajor) {
        return dia_rows<T, SLOTS, SYM>(tr, n, col, vf, gf, cf, of, rf, pre, post);
    } else {
    constexpr int R = round_for(SLOTS, ROUND);
    constexpr bool kDiag = CM == kColDiag;
    const int tid = threadIdx.x;
    auto rows_of = [&](int64_t tt) -> int {
        const int64_t left = n - tt * kTileRows;
        return left < kTileRows ? (int)left : kTileRows;
    };
    int64_t t = tr.first;
    int cur = 0;
    if (t < tr.end) {
        const int rows = rows_of(t);
        if (tid < rows) sm.rp[0][tid] = rp[t * kTileRows + tid];
        if (tid == 0) sm.rp[0][rows] = rp[t * kTileRows + rows];
    }
    if (kDiag && tid < kMaxDiags) sm.dtab[tid] = col.dlt[tid];
    pre();
    __syncthreads();
    if (!post()) return false;
    for (; t < tr.end; t += tr.stride) {
        const int64_t row0 = t * kTileRows;
        const int rows = rows_of(t);
        const IT *cr = sm.rp[cur];
        const int64_t tn = t + tr.stride;
        const bool has_next = tn < tr.end;
        const int rows_n = has_next ? rows_of(tn) : 0;
        IT nrp = 0, nend = 0;
        if (has_next) {
            nrp = rp[tn * kTileRows + (tid < rows_n ? tid : rows_n - 1)];
            nend = rp[tn * kTileRows + rows_n];
        }
        const int me = tid < rows ? tid : rows - 1;
        const auto own = of(row0 + me);
        const uint32_t mk = kDiag ? (uint32_t)col.msk[row0 + me] : 0u;
        const IT base = cr[0];
        const int64_t cnt = (int64_t)(cr[rows] - base);
        // (a diagonal-mask pattern has rows of at most 8 entries: never a plan)
        const bool planned = !kDiag && plan_tiles && plan_tiles[t];
        const bool staged = !planned && cnt > 0 && cnt <= kCap;
        if (staged) {
            const int last = (int)cnt - 1;
            T v[kEpt];
            int32_t c[kEpt];
#pragma unroll
            for (int j = 0; j < kEpt; ++j) {
                const int e = tid + j * kBlock;
                const IT k = base + (e < last ? e : last);
                v[j] = vf(k);
                if (!kDiag) c[j] = col(k, row0);
            }
#pragma unroll
            for (int j = 0; j < kEpt; ++j) {
                sm.val[tid + j * kBlock] = v[j];
                if (!kDiag) sm.col[tid + j * kBlock] = c[j];
            }
        }
        if (has_next) {
            if (tid < rows_n) sm.rp[cur ^ 1][tid] = nrp;
            if (tid == 0) sm.rp[cur ^ 1][rows_n] = nend;
        }
        __syncthreads();
        if (staged) {
            if (tid < rows) {
                const int lo = (int)(cr[tid] - base);
                const int len = (int)(cr[tid + 1] - cr[tid]);
                const int lastk = len > 0 ? len - 1 : 0;
                // columns are ascending and the diagonal is stored, so its
                // position is the number of the row's columns below the row
                const int32_t me32 = (int32_t)(row0 + tid);
                int below = kDiag ? __builtin_popcount(mk & ((1u << col.nneg) - 1u)) : 0;
                uint32_t mm = mk;  // diagonals still to visit (kColDiag)
                T s = T(0);
#pragma unroll
                for (int h = 0; h < SLOTS; h += R) {
                    decltype(gf(0)) g[R];
                    T w[R];
#pragma unroll
                    for (int k = 0; k < R; ++k) {
                        const int idx = lo + (h + k < lastk ? h + k : lastk);
                        int32_t c;
                        if (kDiag) {
                            // slot h + k is the row's (h + k)-th diagonal; past
                            // the row the last one repeats, like the entries
                            c = me32 + sm.dtab[__builtin_ctz(mm | 0x8000u)];
                            mm = h + k < lastk ? (mm & (mm - 1u)) : mm;
                        } else {
                            c = sm.col[idx];
                            below += (h + k < len && c < me32) ? 1 : 0;
                        }
                        w[k] = sm.val[idx];
                        g[k] = gf(c);
                    }
#pragma unroll
                    for (int k = 0; k < R; ++k) {
                        const T sk = fma(w[k], cf(g[k]), s);
                        s = h + k < len ? sk : s;
                    }
                }
                for (int k = SLOTS; k < len; ++k) {
                    const int32_t c = kDiag ? me32 + sm.dtab[nth_bit(mk, k)] : sm.col[lo + k];
                    if (!kDiag) below += c < me32 ? 1 : 0;
                    s = fma(sm.val[lo + k], cf(gf(c)), s);
                }
                rf(row0 + tid, s, own, sm.val[lo + (below < lastk ? below : lastk)]);
            }
        } else if (!planned) {
            const int lane = tid & 63, wave = tid >> 6;
            T *ps = sm.val;              // row sums
            T *pd = sm.val + kTileRows;  // diagonal entries
            for (int r = wave; r < rows; r += kWaves) {
                const IT hi = cr[r + 1];
                const int64_t row = row0 + r;
                T s = T(0);
                const uint32_t mr = kDiag ? (uint32_t)col.msk[row] : 0u;
                for (IT k = cr[r] + lane; k < hi; k += 64) {
                    const int32_t c = kDiag ? (int32_t)row + sm.dtab[nth_bit(mr, (int)(k - cr[r]))]
                                            : col(k, row0);
                    const T v = vf(k);
                    s = fma(v, cf(gf(c)), s);
                    if (c == row) pd[r] = v;  // one lane: the diagonal is stored once
                }
                s = wave_sum_t(s);
                if (lane == 0) ps[r] = s;
            }
            __syncthreads();
            if (tid < rows) rf(row0 + tid, ps[tid], own, pd[tid]);
        }
        __syncthreads();
        cur ^= 1;
    }
    return true;
    }
}

#define SLA_DISPATCH_CM(cm, ...)                    \
    if ((cm) == kColDiag) {                         \
        constexpr int kC = kColDiag;                \
        __VA_ARGS__;                                \
    } else if ((cm) == kColTile16) {                \
        constexpr int kC = kColTile16;              \
        __VA_ARGS__;                                \
    } else {                                        \
        constexpr int kC = kColWide;                \
        __VA_ARGS__;                                \
    }

#define SLA_DISPATCH_SLOTS(slots, ...)                          \
    switch (slots) {                                            \
        case 4: { constexpr int kS = 4; __VA_ARGS__; } break;   \
        case 6: { constexpr int kS = 6; __VA_ARGS__; } break;   \
        default: { constexpr int kS = 8; __VA_ARGS__; } break;  \
    }

// Form of a solver-iteration kernel: kC the column mode, kS the gather slots
// (CSR forms) or the diagonal count 3, 5 or 7 (kColDiaMajor).
#define SLA_DISPATCH_FORM(cm, slots, ...)                           \
    if ((cm) == kColDiaMajor) {                                     \
        constexpr int kC = kColDiaMajor;                            \
        switch (slots) {                                            \
            case 3: { constexpr int kS = 3; __VA_ARGS__; } break;   \
            case 5: { constexpr int kS = 5; __VA_ARGS__; } break;   \
            default: { constexpr int kS = 7; __VA_ARGS__; } break;  \
        }                                                           \
    } else {                                                        \
        SLA_DISPATCH_CM(cm, SLA_DISPATCH_SLOTS(slots, __VA_ARGS__)) \
    }

}  // namespace sla
