// Vector kernels of the Lanczos eigensolver and the eigenvalue gradient.
//
// torch-sla explainer, Methodology section 1 (.eigsh in the autograd-aware
// API) and section 2, eigenvalue problems: the gradient of a simple
// eigenvalue lambda of a symmetric A with unit eigenvector v is
// dlambda/dA_ij = v_i v_j (Hellmann-Feynman), an outer product restricted to
// the stored pattern.
//
// The Lanczos driver (capi.hip) keeps its basis V [m + 1][n] on the device
// and its scalars (alpha, beta, projection coefficients) in a device array,
// so one Lanczos step launches without waiting for the host:
//   dots:    partial sums of V_j . w for a run of basis vectors (grid
//            [blocks][count]), then a fixed-order sum per vector;
//   update:  w -= sum_j c_j V_j with the coefficients read from the device;
//   scale:   V_{j+1} = w / beta_j (zero when beta_j is below the breakdown
//            threshold, which the host detects when it reads the scalars).
#include "sla_internal.h"

namespace sla {

constexpr int kEigBlocks = 256;  // blocks per dot-product pass

// part[j * nb + b] = sum over block b's rows of V_j[i] * w[i]
template <typename T>
__global__ __launch_bounds__(kBlock) void eig_dots_kernel(const T *__restrict__ V, int64_t n,
                                                          const T *__restrict__ w,
                                                          double *__restrict__ part) {
    const int j = blockIdx.y;
    const T *v = V + (int64_t)j * n;
    double acc = 0.0;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride)
        acc += (double)v[i] * (double)w[i];
    __shared__ double red[kWaves];
    acc = wave_sum(acc);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        double s = 0.0;
        for (int k = 0; k < kWaves; ++k) s += red[k];
        part[(int64_t)j * gridDim.x + blockIdx.x] = s;
    }
}

// out[j] = sum of the nb partials of vector j in block order (sqrt when
// `root`): one block per vector, identical result on every run.
__global__ __launch_bounds__(kBlock) void eig_sum_kernel(const double *__restrict__ part, int nb,
                                                         double *__restrict__ out, int root) {
    const int j = blockIdx.x;
    double acc = 0.0;
    for (int b = threadIdx.x; b < nb; b += kBlock) acc += part[(int64_t)j * nb + b];
    __shared__ double red[kWaves];
    acc = wave_sum(acc);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        double s = 0.0;
        for (int k = 0; k < kWaves; ++k) s += red[k];
        out[j] = root ? sqrt(s) : s;
    }
}

// w[i] -= sum_{j < m} c[j] * V_j[i]
template <typename T>
__global__ __launch_bounds__(kBlock) void eig_update_kernel(T *__restrict__ w,
                                                            const T *__restrict__ V, int m,
                                                            const double *__restrict__ c,
                                                            int64_t n) {
    extern __shared__ double cs[];
    for (int j = threadIdx.x; j < m; j += kBlock) cs[j] = c[j];
    __syncthreads();
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride) {
        double acc = 0.0;
        for (int j = 0; j < m; ++j) acc += cs[j] * (double)V[(int64_t)j * n + i];
        w[i] = (T)((double)w[i] - acc);
    }
}

// out = w / beta (0 when beta <= tiny: an invariant subspace was found)
template <typename T>
__global__ __launch_bounds__(kBlock) void eig_scale_kernel(const T *__restrict__ w,
                                                           T *__restrict__ out,
                                                           const double *__restrict__ beta,
                                                           double tiny, int64_t n) {
    const double b = *beta;
    const double r = b > tiny ? 1.0 / b : 0.0;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride)
        out[i] = (T)((double)w[i] * r);
}

// X_i = sum_j S[j * k + i] V_j for i < k (Ritz vectors; S on the device)
template <typename T>
__global__ __launch_bounds__(kBlock) void eig_combine_kernel(T *__restrict__ X,
                                                             const T *__restrict__ V, int m,
                                                             int k, const double *__restrict__ S,
                                                             int64_t n) {
    extern __shared__ double ss[];
    for (int j = threadIdx.x; j < m * k; j += kBlock) ss[j] = S[j];
    __syncthreads();
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride)
        for (int q = 0; q < k; ++q) {
            double acc = 0.0;
            for (int j = 0; j < m; ++j) acc += ss[j * k + q] * (double)V[(int64_t)j * n + i];
            X[(int64_t)q * n + i] = (T)acc;
        }
}

// grad[e] = sum_q g[q] * X_q[row(e)] * X_q[col(e)] for every stored entry:
// the eigenvalue gradient on the pattern for upstream weights g.
template <typename T, typename IT>
__global__ __launch_bounds__(kBlock) void eig_outer_kernel(const IT *__restrict__ rp,
                                                           const int32_t *__restrict__ col,
                                                           const T *__restrict__ X, int k,
                                                           const T *__restrict__ g,
                                                           T *__restrict__ grad, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride) {
        for (IT e = rp[i]; e < rp[i + 1]; ++e) {
            const int32_t c = col[e];
            T acc = T(0);
            for (int q = 0; q < k; ++q) acc += g[q] * X[(int64_t)q * n + i] * X[(int64_t)q * n + c];
            grad[e] = acc;
        }
    }
}

// ------------------------------------------------------------------ launchers

static unsigned eig_blocks(int64_t n) {
    int64_t b = (n + kBlock - 1) / kBlock;
    if (b > 4096) b = 4096;
    if (b < 1) b = 1;
    return (unsigned)b;
}

template <typename T>
hipError_t launch_eig_dots(const T *V, int m, const T *w, int64_t n, double *part, double *out,
                           bool root, hipStream_t s) {
    int64_t nb = (n + kBlock - 1) / kBlock;
    if (nb > kEigBlocks) nb = kEigBlocks;
    if (nb < 1) nb = 1;
    eig_dots_kernel<T><<<dim3((unsigned)nb, m), kBlock, 0, s>>>(V, n, w, part);
    eig_sum_kernel<<<m, kBlock, 0, s>>>(part, (int)nb, out, root ? 1 : 0);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_eig_update(T *w, const T *V, int m, const double *c, int64_t n, hipStream_t s) {
    eig_update_kernel<T><<<eig_blocks(n), kBlock, sizeof(double) * m, s>>>(w, V, m, c, n);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_eig_scale(const T *w, T *out, const double *beta, double tiny, int64_t n,
                            hipStream_t s) {
    eig_scale_kernel<T><<<eig_blocks(n), kBlock, 0, s>>>(w, out, beta, tiny, n);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_eig_combine(T *X, const T *V, int m, int k, const double *S, int64_t n,
                              hipStream_t s) {
    eig_combine_kernel<T><<<eig_blocks(n), kBlock, sizeof(double) * m * k, s>>>(X, V, m, k, S, n);
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_eig_outer(const IT *rp, const int32_t *col, const T *X, int k, const T *g,
                            T *grad, int64_t n, hipStream_t s) {
    eig_outer_kernel<T, IT><<<eig_blocks(n), kBlock, 0, s>>>(rp, col, X, k, g, grad, n);
    return hipGetLastError();
}

#define SLA_EIG_T(T)                                                                            \
    template hipError_t launch_eig_dots<T>(const T *, int, const T *, int64_t, double *,        \
                                           double *, bool, hipStream_t);                        \
    template hipError_t launch_eig_update<T>(T *, const T *, int, const double *, int64_t,      \
                                             hipStream_t);                                      \
    template hipError_t launch_eig_scale<T>(const T *, T *, const double *, double, int64_t,    \
                                            hipStream_t);                                       \
    template hipError_t launch_eig_combine<T>(T *, const T *, int, int, const double *,         \
                                              int64_t, hipStream_t);
SLA_EIG_T(float)
SLA_EIG_T(double)
template hipError_t launch_eig_outer<float, int32_t>(const int32_t *, const int32_t *,
                                                     const float *, int, const float *, float *,
                                                     int64_t, hipStream_t);
template hipError_t launch_eig_outer<float, int64_t>(const int64_t *, const int32_t *,
                                                     const float *, int, const float *, float *,
                                                     int64_t, hipStream_t);
template hipError_t launch_eig_outer<double, int32_t>(const int32_t *, const int32_t *,
                                                      const double *, int, const double *,
                                                      double *, int64_t, hipStream_t);
template hipError_t launch_eig_outer<double, int64_t>(const int64_t *, const int32_t *,
                                                      const double *, int, const double *,
                                                      double *, int64_t, hipStream_t);

}  // namespace sla
