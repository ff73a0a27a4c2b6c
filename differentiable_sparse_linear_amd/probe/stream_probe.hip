// Bandwidth ceilings of the chip, measured by the benchmark beside the
// solver kernels (libsla_probe.so; not part of the solver library).
//
//   read   sum of a[0..n) (each element read once; one partial per block)
//   copy   b = a
//   write  b = v
//   copy_passes  b = a + 1, a = b + 1, ... over arrays that stay in the
//          256 MB Infinity Cache, one launch (the in-cache copy ceiling)
//   streams  R arrays read and W written at once, in the cache, one launch
//          per pass (the shape of a grid iteration kernel)
//   lds    workgroups (two resident per compute unit) each read their own
//          64 KB of LDS over and over
//
// The streaming kernels move 16 bytes per thread and access with eight
// independent accesses in flight per thread; grids fill all 256 compute units
// many times over.  Their byte counts are
// exact, so the read kernel also serves as a known-traffic reference for the
// hardware counters next to the copy.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sla_probe.h"

namespace {

typedef double v2d __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kBlocks = 256 * 128;  // 128 workgroups per compute unit
constexpr int kUnroll = 8;

// Non-temporal loads and stores: each element is touched once, so the
// lines need not stay in the caches (measured on MI355X over 4 GiB arrays:
// read 7.0 TB/s with them, 6.2 without; copy 5.4 and 5.2).
__device__ __forceinline__ v2d ld(const v2d *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st(v2d v, v2d *p) { __builtin_nontemporal_store(v, p); }

__global__ __launch_bounds__(kThreads) void read_kernel(const v2d *__restrict__ a, int64_t n2,
                                                        double *__restrict__ part) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    double s[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) s[u] = 0.0;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    for (; i + (kUnroll - 1) * stride < n2; i += kUnroll * stride) {
        v2d x[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) x[u] = ld(&a[i + u * stride]);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) s[u] += x[u].x + x[u].y;
    }
    for (; i < n2; i += stride) s[0] += a[i].x + a[i].y;
    double t = 0.0;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) t += s[u];
    for (int off = 32; off > 0; off >>= 1) t += __shfl_xor(t, off, 64);
    __shared__ double w[kThreads / 64];
    if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = t;
    __syncthreads();
    if (threadIdx.x == 0) part[blockIdx.x] = (w[0] + w[1]) + (w[2] + w[3]);
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const v2d *__restrict__ a,
                                                        v2d *__restrict__ b, int64_t n2) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    for (; i + (kUnroll - 1) * stride < n2; i += kUnroll * stride) {
        v2d x[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) x[u] = ld(&a[i + u * stride]);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) st(x[u], &b[i + u * stride]);
    }
    for (; i < n2; i += stride) b[i] = a[i];
}

__global__ __launch_bounds__(kThreads) void write_kernel(v2d *__restrict__ b, int64_t n2,
                                                         double v) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const v2d x = {v, v};
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n2; i += stride)
        st(x, &b[i]);
}

// In-cache copy: `passes` passes over two arrays of n2 16-byte elements,
// small enough to stay in the Infinity Cache, with plain accesses so that
// their lines stay there; pass p reads one array and writes the other.  A
// thread touches the same elements in every pass, so the passes need no
// barrier between them, and each pass's values depend on the last one's.
constexpr int kPassBlocks = 256 * 8;  // eight workgroups per compute unit

__global__ __launch_bounds__(kThreads) void copy_passes_kernel(v2d *__restrict__ a,
                                                               v2d *__restrict__ b, int64_t n2,
                                                               int32_t passes) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const int64_t i0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    for (int32_t p = 0; p < passes; ++p) {
        const v2d *src = (p & 1) ? b : a;
        v2d *dst = (p & 1) ? a : b;
        int64_t i = i0;
        for (; i + (kUnroll - 1) * stride < n2; i += kUnroll * stride) {
            v2d x[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) x[u] = src[i + u * stride];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) dst[i + u * stride] = x[u] + 1.0;
        }
        for (; i < n2; i += stride) dst[i] = src[i] + 1.0;
    }
}

// Many streams at once, in the cache: R arrays read and W arrays written per
// launch, n2 16-byte elements each, consecutive in one buffer; element i of
// every written array gets the sum of element i of the read ones (plus its
// index).  768 workgroups of 256 threads, plain accesses, one launch per
// pass: the shape of a grid iteration kernel that reads and writes many
// vectors of a system that stays in the Infinity Cache.
constexpr int kStreamBlocks = 768;

template <int R, int W>
__global__ __launch_bounds__(kThreads) void streams_kernel(v2d *__restrict__ buf, int64_t n2) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n2; i += stride) {
        v2d x[R];
#pragma unroll
        for (int r = 0; r < R; ++r) x[r] = buf[r * n2 + i];
        v2d t = x[0];
#pragma unroll
        for (int r = 1; r < R; ++r) t += x[r];
#pragma unroll
        for (int w = 0; w < W; ++w) buf[(R + w) * n2 + i] = t + (double)w;
    }
}

// LDS reads: thread t reads 16 bytes at a rotating offset of a 64 KB block
// of LDS (consecutive lanes take consecutive 16-byte words, no bank
// conflicts); the sum keeps the reads alive.
constexpr int kLdsWords = 65536 / 16;
constexpr int kLdsBlocks = 256 * 8;  // two of 64 KB at a time per compute unit, four rounds

__global__ __launch_bounds__(1024) void lds_kernel(int64_t reps, double *__restrict__ part) {
    __shared__ double2 buf[kLdsWords];
    for (int j = threadIdx.x; j < kLdsWords; j += blockDim.x)
        buf[j] = make_double2((double)j, 1.0);
    __syncthreads();
    double s0 = 0.0, s1 = 0.0;
    int o = threadIdx.x;
    for (int64_t r = 0; r < reps; ++r) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const double2 x = buf[(o + k * 1024) & (kLdsWords - 1)];
            s0 += x.x;
            s1 += x.y;
        }
        o = (o + 64) & (kLdsWords - 1);
    }
    const double s = s0 + s1;
    if (s == -1.0) part[blockIdx.x] = s;  // never true; keeps the loads
}

}  // namespace

extern "C" {

int32_t sla_probe_blocks(void) { return kBlocks; }

int32_t sla_probe_read(const void *d_a, int64_t n, void *d_part, void *stream) {
    if (!d_a || !d_part || n < 2 || (n & 1)) return -1;
    read_kernel<<<kBlocks, kThreads, 0, reinterpret_cast<hipStream_t>(stream)>>>(
        reinterpret_cast<const v2d *>(d_a), n / 2, reinterpret_cast<double *>(d_part));
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

int32_t sla_probe_copy(const void *d_a, void *d_b, int64_t n, void *stream) {
    if (!d_a || !d_b || n < 2 || (n & 1)) return -1;
    copy_kernel<<<kBlocks, kThreads, 0, reinterpret_cast<hipStream_t>(stream)>>>(
        reinterpret_cast<const v2d *>(d_a), reinterpret_cast<v2d *>(d_b), n / 2);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

int32_t sla_probe_write(void *d_b, int64_t n, double v, void *stream) {
    if (!d_b || n < 2 || (n & 1)) return -1;
    write_kernel<<<kBlocks, kThreads, 0, reinterpret_cast<hipStream_t>(stream)>>>(
        reinterpret_cast<v2d *>(d_b), n / 2, v);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

int32_t sla_probe_copy_passes(void *d_a, void *d_b, int64_t n, int32_t passes, void *stream) {
    if (!d_a || !d_b || n < 2 || (n & 1) || passes < 1) return -1;
    copy_passes_kernel<<<kPassBlocks, kThreads, 0, reinterpret_cast<hipStream_t>(stream)>>>(
        reinterpret_cast<v2d *>(d_a), reinterpret_cast<v2d *>(d_b), n / 2, passes);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

int32_t sla_probe_streams(void *d_buf, int64_t n, int32_t reads, int32_t writes,
                          void *stream) {
    if (!d_buf || n < 2 || (n & 1)) return -1;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    v2d *b = reinterpret_cast<v2d *>(d_buf);
    const int64_t n2 = n / 2;
    if (reads == 2 && writes == 2)
        streams_kernel<2, 2><<<kStreamBlocks, kThreads, 0, s>>>(b, n2);
    else if (reads == 8 && writes == 4)
        streams_kernel<8, 4><<<kStreamBlocks, kThreads, 0, s>>>(b, n2);
    else if (reads == 9 && writes == 5)
        streams_kernel<9, 5><<<kStreamBlocks, kThreads, 0, s>>>(b, n2);
    else if (reads == 12 && writes == 4)
        streams_kernel<12, 4><<<kStreamBlocks, kThreads, 0, s>>>(b, n2);
    else
        return -1;
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

int64_t sla_probe_lds(int64_t reps, void *d_part, void *stream) {
    if (!d_part || reps < 1) return -1;
    lds_kernel<<<kLdsBlocks, 1024, 0, reinterpret_cast<hipStream_t>(stream)>>>(
        reps, reinterpret_cast<double *>(d_part));
    if (hipGetLastError() != hipSuccess) return -5;
    return (int64_t)kLdsBlocks * 1024 * reps * 4 * 16;  // bytes read from LDS
}

}  // extern "C"
