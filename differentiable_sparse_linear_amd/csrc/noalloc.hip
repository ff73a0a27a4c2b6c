// sla_solve_noalloc: the forward CG solve of small systems with no handle and
// no allocation, for callers that cannot allocate device memory.
//
// It runs the one-workgroup CG solver that sla_solve uses for systems of at
// most kBlockSolveMaxN rows (vectors in LDS), so its results are those of
// sla_solve bit for bit.  What sla_solve keeps in the handle -- the
// diagonal index, the per-system SolveState, the validation flags -- lives
// here in one file-scope device array, `scratch`, of a fixed size.  Each
// device holds its own copy of the array at its own address; the host
// takes that address once per device with hipGetSymbolAddress and uses
// only it (the array's name is a host-side stand-in, not a device
// address).  Every call on a device shares its copy, so calls that overlap
// on one device race.
#include <math.h>

#include <mutex>
#include <type_traits>

#include "sla_internal.h"

namespace sla {
namespace {

constexpr int64_t kNaMaxN = kBlockSolveMaxN;  // rows per system
constexpr int64_t kNaMaxBatch = 65535;        // systems per call (one launch)

constexpr int64_t na_align(int64_t b) { return (b + 255) / 256 * 256; }

// Layout of the scratch array, in bytes.
constexpr int64_t kNaHdr = 0;  // int32 [4]: flag, longest row, worst status < 0, worst > 0
constexpr int64_t kNaDiag = 256;                                           // IT [n]
constexpr int64_t kNaState = kNaDiag + na_align(kNaMaxN * 8);              // SolveState [B]
constexpr int64_t kNaIters = kNaState + na_align(kNaMaxBatch * (int64_t)sizeof(SolveState));
constexpr int64_t kNaSpmv = kNaIters + na_align(kNaMaxBatch * 4);          // int32 [B]
constexpr int64_t kNaStatus = kNaSpmv + na_align(kNaMaxBatch * 4);         // int32 [B]
constexpr int64_t kNaRelres = kNaStatus + na_align(kNaMaxBatch * 4);       // double [B]
constexpr int64_t kNaBytes = kNaRelres + na_align(kNaMaxBatch * 8);
static_assert(kNaBytes <= ((int64_t)16 << 20), "the scratch array stays modest");

}  // namespace

static __device__ __align__(256) unsigned char scratch[kNaBytes];

namespace {

constexpr int kNaMaxDevices = 64;
std::mutex g_na_mutex;
unsigned char *g_na_ptr[kNaMaxDevices] = {};

// The device address of the current device's scratch array, taken on the
// first call on that device.
hipError_t scratch_of_device(unsigned char **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kNaMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_na_mutex);
    if (!g_na_ptr[dev]) {
        void *p = nullptr;
        if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
        g_na_ptr[dev] = static_cast<unsigned char *>(p);
    }
    *out = g_na_ptr[dev];
    return hipSuccess;
}

__global__ __launch_bounds__(64) void na_clear_kernel(int32_t *hdr) {
    if (threadIdx.x < 4) hdr[threadIdx.x] = 0;
}

// Per-system results from the states, and the most severe statuses (hdr[2]:
// the lowest negative, hdr[3]: the highest positive), one atomic per
// wavefront.
__global__ __launch_bounds__(kBlock) void na_report_kernel(const SolveState *st, int64_t batch,
                                                          int32_t *iters, int32_t *spmv,
                                                          int32_t *status, double *relres,
                                                          int32_t *hdr) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    int neg = 0, pos = 0;
    if (i < batch) {
        const SolveState s = st[i];
        iters[i] = s.iter;
        spmv[i] = s.spmv;
        status[i] = s.status;
        relres[i] = s.bb > 0.0 ? sqrt(s.rr) / sqrt(s.bb) : 0.0;
        neg = s.status < 0 ? s.status : 0;
        pos = s.status > 0 ? s.status : 0;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const int a = __shfl_xor(neg, off, 64), b = __shfl_xor(pos, off, 64);
        neg = a < neg ? a : neg;
        pos = b > pos ? b : pos;
    }
    if ((threadIdx.x & 63) == 0) {
        if (neg < 0) atomicMin(&hdr[2], neg);
        if (pos > 0) atomicMax(&hdr[3], pos);
    }
}

#define NA_TRY(...)                    \
    do {                               \
        hipError_t e_ = (__VA_ARGS__); \
        if (e_ != hipSuccess) {        \
            set_last_error(e_);        \
            return SLA_ERR_DEVICE;     \
        }                              \
    } while (0)

template <typename T, typename IT>
sla_status solve_noalloc(unsigned char *base, int64_t n, int64_t nnz, int64_t batch,
                         const IT *rp, const int32_t *col, const T *val, const T *b, T *x,
                         const sla_solve_opts &o, sla_solve_info *info, hipStream_t s) {
    int32_t *hdr = reinterpret_cast<int32_t *>(base + kNaHdr);
    IT *diagpos = reinterpret_cast<IT *>(base + kNaDiag);
    SolveState *st = reinterpret_cast<SolveState *>(base + kNaState);
    int32_t *iters = reinterpret_cast<int32_t *>(base + kNaIters);
    int32_t *spmv = reinterpret_cast<int32_t *>(base + kNaSpmv);
    int32_t *status = reinterpret_cast<int32_t *>(base + kNaStatus);
    double *relres = reinterpret_cast<double *>(base + kNaRelres);
    int32_t h[4] = {0, 0, 0, 0};
    // the flags and the longest row start at 0 (the array keeps the last
    // call's contents)
    na_clear_kernel<<<1, 64, 0, s>>>(hdr);
    NA_TRY(hipGetLastError());
    // the row pointers first: the column checks read col[rp[i]..rp[i+1])
    NA_TRY(launch_check_rowptr<IT>(rp, n, nnz, &hdr[0], s));
    NA_TRY(hipMemcpyAsync(h, hdr, sizeof(int32_t), hipMemcpyDeviceToHost, s));
    NA_TRY(hipStreamSynchronize(s));
    if (h[0]) return SLA_ERR_PATTERN;
    NA_TRY(launch_max_row<IT>(rp, n, &hdr[1], s));
    NA_TRY(launch_check_cols_rows<IT>(rp, col, n, diagpos, &hdr[0], s));
    NA_TRY(hipMemcpyAsync(h, hdr, 2 * sizeof(int32_t), hipMemcpyDeviceToHost, s));
    NA_TRY(hipStreamSynchronize(s));
    if (h[0]) return SLA_ERR_PATTERN;
    BlockCgParams p;
    p.val = val;
    p.rp = rp;
    p.col = col;
    p.diagpos = diagpos;
    p.x = x;
    p.b = b;
    p.st = st;
    p.n = n;
    p.nnz = nnz;
    p.tol = o.tol;
    p.maxit = o.maxit;
    p.use_x0 = o.use_x0;
    p.jac = o.precond == SLA_PRECOND_JACOBI;
    NA_TRY((launch_block_cg<T, IT>(h[1], p, (int)batch, s)));
    const unsigned nb = (unsigned)((batch + kBlock - 1) / kBlock);
    na_report_kernel<<<nb, kBlock, 0, s>>>(st, batch, iters, spmv, status, relres, hdr);
    NA_TRY(hipGetLastError());
    if (info) {
        if (info->iters)
            NA_TRY(hipMemcpyAsync(info->iters, iters, 4 * batch, hipMemcpyDeviceToHost, s));
        if (info->spmv)
            NA_TRY(hipMemcpyAsync(info->spmv, spmv, 4 * batch, hipMemcpyDeviceToHost, s));
        if (info->status)
            NA_TRY(hipMemcpyAsync(info->status, status, 4 * batch, hipMemcpyDeviceToHost, s));
        if (info->relres)
            NA_TRY(hipMemcpyAsync(info->relres, relres, 8 * batch, hipMemcpyDeviceToHost, s));
        info->kernel_ms = 0.0;
        info->kernel_launches = 0;
        info->form = -1;
    }
    NA_TRY(hipMemcpyAsync(h, hdr, 4 * sizeof(int32_t), hipMemcpyDeviceToHost, s));
    NA_TRY(hipStreamSynchronize(s));
    return (sla_status)(h[2] < 0 ? h[2] : h[3]);
}

}  // namespace
}  // namespace sla

using namespace sla;

extern "C" {

sla_status sla_solve_noalloc(int64_t n, int64_t nnz, int64_t batch, int32_t dtype,
                             int32_t row_ptr_type, const void *d_row_ptr, const int32_t *d_col,
                             const void *d_values, const void *d_b, void *d_x,
                             const sla_solve_opts *opts, sla_solve_info *info, void *stream) {
    if (n < 1 || nnz < n || batch < 1) return SLA_ERR_ARG;
    if (n > kNaMaxN || batch > kNaMaxBatch) return SLA_ERR_TOO_LARGE;
    if (nnz >= ((int64_t)1 << 31)) return SLA_ERR_ARG;
    if (dtype != SLA_F32 && dtype != SLA_F64) return SLA_ERR_ARG;
    if (row_ptr_type != SLA_I32 && row_ptr_type != SLA_I64) return SLA_ERR_ARG;
    if (!d_row_ptr || !d_col || !d_values || !d_b || !d_x || d_b == d_x) return SLA_ERR_ARG;
    sla_solve_opts o;
    o.tol = 1e-10;
    o.maxit = 1000;
    o.method = SLA_CG;
    o.precond = SLA_PRECOND_JACOBI;
    o.use_x0 = 0;
    o.graph_chunk = 0;
    o.profile = 0;
    if (opts) o = *opts;
    if (!(o.tol >= 0.0) || o.maxit < 0 || o.method != SLA_CG || o.profile != 0) return SLA_ERR_ARG;
    if (o.precond != SLA_PRECOND_NONE && o.precond != SLA_PRECOND_JACOBI) return SLA_ERR_ARG;
    unsigned char *base = nullptr;
    if (hipError_t e = scratch_of_device(&base); e != hipSuccess) {
        set_last_error(e);
        return SLA_ERR_DEVICE;
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    auto run = [&](auto t, auto it) -> sla_status {
        using T = std::remove_pointer_t<decltype(t)>;
        using IT = std::remove_pointer_t<decltype(it)>;
        return solve_noalloc<T, IT>(base, n, nnz, batch, reinterpret_cast<const IT *>(d_row_ptr),
                                    d_col, reinterpret_cast<const T *>(d_values),
                                    reinterpret_cast<const T *>(d_b), reinterpret_cast<T *>(d_x),
                                    o, info, s);
    };
    if (dtype == SLA_F64)
        return row_ptr_type == SLA_I64 ? run((double *)nullptr, (int64_t *)nullptr)
                                       : run((double *)nullptr, (int32_t *)nullptr);
    return row_ptr_type == SLA_I64 ? run((float *)nullptr, (int64_t *)nullptr)
                                   : run((float *)nullptr, (int32_t *)nullptr);
}

}  // extern "C"
