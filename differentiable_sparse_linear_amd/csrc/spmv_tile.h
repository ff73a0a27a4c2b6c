// One tile of a CSR product, shared by every SpMV-shaped grid kernel.
//
// A tile is kTileRows consecutive rows.  Their entries form one contiguous
// run [rp[row0], rp[row0 + rows]) of the value and column arrays, so the
// block reads that run as consecutive elements (entry e by thread e mod
// kBlock, kEpt entries per thread, all loads independent and issued before
// any is used), multiplies each value by the gathered vector entry, and
// stages the products in LDS.  After a barrier each thread adds the products
// of one row in entry order.  A tile with more than kBlock * kEpt entries
// (long rows) is processed one wavefront per row instead, lanes striding over
// the row's entries.
#pragma once

#include "sla_internal.h"

namespace sla {

constexpr int kEpt = 8;                  // staged entries per thread
constexpr int kCap = kBlock * kEpt;      // staged entries per tile

template <typename T, typename IT>
struct TileLds {
    IT rp[kTileRows + 1];
    T prod[kCap];
};

__device__ __forceinline__ float wave_sum_t(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}
__device__ __forceinline__ double wave_sum_t(double v) { return wave_sum(v); }

// vf(k): value of stored entry k; xf(c): vector entry gathered at column c;
// rf(i, s): consumes row i's product s (called once per row of the tile).
template <typename T, typename IT, typename VF, typename XF, typename RF>
__device__ __forceinline__ void spmv_tile(int64_t t, int64_t n, const IT *__restrict__ rp,
                                          const int32_t *__restrict__ col, TileLds<T, IT> &sm,
                                          VF vf, XF xf, RF rf) {
    const int tid = threadIdx.x;
    const int64_t row0 = t * kTileRows;
    const int64_t left = n - row0;
    const int rows = left < kTileRows ? (int)left : kTileRows;
    if (tid < rows) sm.rp[tid] = rp[row0 + tid];
    if (tid == 0) sm.rp[rows] = rp[row0 + rows];
    __syncthreads();
    const IT base = sm.rp[0];
    const int64_t cnt = (int64_t)(sm.rp[rows] - base);
    if (cnt <= kCap) {
        T v[kEpt], xv[kEpt];
        int32_t c[kEpt];
#pragma unroll
        for (int j = 0; j < kEpt; ++j) {
            const int e = tid + j * kBlock;
            if (e < cnt) {
                v[j] = vf(base + e);
                c[j] = col[base + e];
            }
        }
#pragma unroll
        for (int j = 0; j < kEpt; ++j) {
            const int e = tid + j * kBlock;
            if (e < cnt) xv[j] = xf(c[j]);
        }
#pragma unroll
        for (int j = 0; j < kEpt; ++j) {
            const int e = tid + j * kBlock;
            if (e < cnt) sm.prod[e] = v[j] * xv[j];
        }
        __syncthreads();
        if (tid < rows) {
            const int lo = (int)(sm.rp[tid] - base), hi = (int)(sm.rp[tid + 1] - base);
            T s = T(0);
            for (int e = lo; e < hi; ++e) s += sm.prod[e];
            rf(row0 + tid, s);
        }
    } else {
        const int lane = tid & 63, wave = tid >> 6;
        for (int r = wave; r < rows; r += kWaves) {
            const IT hi = sm.rp[r + 1];
            T s = T(0);
            for (IT k = sm.rp[r] + lane; k < hi; k += 64) s += vf(k) * xf(col[k]);
            s = wave_sum_t(s);
            if (lane == 0) rf(row0 + r, s);
        }
    }
    __syncthreads();  // the next tile reuses the LDS
}

}  // namespace sla
