// C ABI of the sparse solve: handle lifetime, workspace, and the drivers that
// enqueue the iteration kernels.
//
// Launch control (torch-sla explainer, Problem statement: iterative solvers
// pay kernel-launch overhead on small problems):
//  * small systems (n <= 4096, short rows) solve with CG in one workgroup per
//    system, a single launch for the whole batch;
//  * larger systems run the grid kernels; K iterations are captured
//    once in a HIP graph that reads its arguments from a device block, every
//    kernel ends at its first barrier once the device-side `done` flag is
//    set, each replay ends by storing the count of stopped systems into
//    pinned host memory, and the host keeps one replay in flight while it
//    reads the count that the previous one left;
//  * CG on a batch of larger systems advances a group of them per launch
//    (the y dimension of the grid), as many as fit kGroupRows rows of
//    workspace, and polls the count of the group's stopped systems.
// Nothing is allocated after sla_create (memory is O(n + nnz) whatever the
// iteration count -- Methodology section 2, complexity bullet).
#include <math.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <type_traits>
#include <vector>

#include "sla_internal.h"

using namespace sla;

namespace {
thread_local hipError_t g_last_error = hipSuccess;
}  // namespace

void sla::set_last_error(hipError_t e) { g_last_error = e; }

namespace {

constexpr int kNumVec = 11;  // r z q rh s t p0 p1 v0 v1 dinv
constexpr int kDefaultChunk = 16;
// Rows per launch (system rows x systems of the group) from which the fused
// iterations are launched directly by default rather than as replays of a
// captured graph: each replay boundary left the GPU idle for about 13 us,
// while from these sizes on the host enqueues launches faster than the GPU
// runs them.  Measured per step of forward + adjoint (MI355X, fp64, chunks of
// 32), CG on 3D diffusion: 4913 rows -2 %, 13 824 -1 %, 32 768 +1.8 %,
// 64 000 +3.9 %, 262 144 +3.5 %, 10^6 +1.2 %; BiCGStab on 2D
// convection-diffusion: 16 384 rows -3 %, 65 536 +0.2 %, 1 048 576 +0.4 %.
constexpr int64_t kDirectRowsCg = (int64_t)1 << 15;
constexpr int64_t kDirectRowsBicg = (int64_t)1 << 16;
// Rows of the systems that one grid CG launch advances together: about
// 2M rows keep a launch's traffic (~190 bytes per row and iteration) two
// orders of magnitude above the launch overhead; the workspace grows with it.
constexpr int64_t kGroupRows = (int64_t)1 << 21;

constexpr int kGraphSlots = 8;

struct GraphEntry {
    int key = -1;
    int chunk = 0;
    hipGraphExec_t exec = nullptr;
};

}  // namespace

struct sla_ctx {
    int device = 0;
    int64_t n = 0, nnz = 0, batch = 0;
    int dtype = SLA_F64, itype = SLA_I32;
    const void *rp = nullptr;
    const int32_t *col = nullptr;
    ColArgs ca, ca_t;            // where the products read the columns of A, A^T
    ColArgs ia, ia_t;            // the form the solver iterations read for A, A^T
    void *dia = nullptr;         // diagonal-major values [gbatch][nd][n], or null
    int32_t *dlt = nullptr;      // [2][kMaxDiags] diagonal offsets of A, A^T
    uint16_t *msk = nullptr;     // per-row diagonal masks of A, or null
    uint16_t *msk_t = nullptr;   // the same for A^T
    int16_t *col16 = nullptr;    // compact columns of A, or null
    void *diagpos = nullptr;
    bool has_t = false;
    void *rp_t = nullptr;
    int32_t *col_t = nullptr;
    int16_t *col16_t = nullptr;  // compact columns of A^T, or null
    int32_t *perm = nullptr;     // A's position of each A^T entry
    int32_t *pinv = nullptr;     // A^T's position of each A entry
    void *val_t = nullptr;       // one system's values (or products) in A^T's order
    int32_t *bpos = nullptr;     // where the terms pass stores each A entry's term (or null)
    uint16_t *lidx = nullptr;    // for the row sums: each such term's offset in its tile
    int slots = 8;   // gather slots per row (A), from its longest row
    int max_len = 0; // longest row of A
    int slots_t = 8; // the same for A^T
    int it_slots = 8, it_slots_t = 8;  // slots (or diagonals) of the iteration form
    RowPlan plan, plan_t;        // tiles past the LDS stage, of A and of A^T (or empty)
    void *plan_mem[2][4] = {};   // their items, split rows, partial sums and tile flags
    int64_t gbatch = 1;          // systems per grid launch
    void *vec = nullptr;         // [kNumVec][gbatch][n]
    SolveState *st = nullptr;
    double *part = nullptr;      // [gbatch][kPartStride]
    int32_t *ndone = nullptr;    // stopped systems of the running launch group
    void *args_dev = nullptr;    // [gbatch] IterArgs, one per system of a launch group
    void *args_host = nullptr;   // pinned staging copy of args_dev
    int32_t *flag = nullptr;
    int32_t *poll = nullptr;     // pinned, coherent [2]: stopped systems
    int32_t *poll_dev = nullptr; // its device address
    SolveState *st_host = nullptr;  // pinned [batch]
    hipStream_t cap = nullptr;
    hipEvent_t ev[2] = {nullptr, nullptr};
    hipStream_t side = nullptr;  // the product backward's gradient pass, beside the A^T passes
    hipEvent_t fork = nullptr, join = nullptr;
    std::vector<hipEvent_t> prof_ev;
    GraphEntry graphs[kGraphSlots];
    int graph_next = 0;          // next slot to replace when all are taken
    int32_t last_iters = 0;      // most iterations of a system in the last grid solve
    int64_t ws_bytes = 0;
    // sla_eigsh's Lanczos basis and scalars, grown to the largest call so far
    void *eig_V = nullptr;       // [(eig_m + 1) * n] values
    double *eig_sc = nullptr;    // alpha, beta, coefficients, Ritz vectors, norm
    double *eig_part = nullptr;  // partial sums
    int eig_m = 0, eig_k = 0;    // basis and eigenpair counts the buffers hold
    int64_t eig_bytes = 0;
};

namespace {

inline size_t tsize(const sla_ctx *h) { return h->dtype == SLA_F64 ? 8 : 4; }

struct DeviceGuard {
    int prev = -1;
    explicit DeviceGuard(int dev) {
        int cur = 0;
        if (hipGetDevice(&cur) == hipSuccess && cur != dev) {
            prev = cur;
            (void)hipSetDevice(dev);
        }
    }
    ~DeviceGuard() {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
};

#define HIP_TRY(...)                          \
    do {                                      \
        hipError_t e_ = (__VA_ARGS__);        \
        if (e_ != hipSuccess) {               \
            g_last_error = e_;                \
            return SLA_ERR_DEVICE;            \
        }                                     \
    } while (0)

template <typename P>
hipError_t dmalloc(sla_ctx *h, P **p, size_t bytes) {
    hipError_t e = hipMalloc((void **)p, bytes > 0 ? bytes : 1);
    if (e == hipSuccess) h->ws_bytes += (int64_t)(bytes > 0 ? bytes : 1);
    return e;
}

void release(sla_ctx *h) {
    if (!h) return;
    for (auto &g : h->graphs)
        if (g.exec) (void)hipGraphExecDestroy(g.exec);
    for (auto e : h->prof_ev) (void)hipEventDestroy(e);
    for (auto e : h->ev)
        if (e) (void)hipEventDestroy(e);
    if (h->cap) (void)hipStreamDestroy(h->cap);
    if (h->side) (void)hipStreamDestroy(h->side);
    if (h->fork) (void)hipEventDestroy(h->fork);
    if (h->join) (void)hipEventDestroy(h->join);
    (void)hipFree(h->diagpos);
    (void)hipFree(h->col16);
    (void)hipFree(h->dlt);
    (void)hipFree(h->msk);
    (void)hipFree(h->msk_t);
    (void)hipFree(h->rp_t);
    (void)hipFree(h->col_t);
    (void)hipFree(h->col16_t);
    (void)hipFree(h->perm);
    (void)hipFree(h->pinv);
    (void)hipFree(h->val_t);
    (void)hipFree(h->bpos);
    (void)hipFree(h->lidx);
    (void)hipFree(h->dia);
    for (auto &pm : h->plan_mem)
        for (void *p : pm) (void)hipFree(p);
    (void)hipFree(h->eig_V);
    (void)hipFree(h->eig_sc);
    (void)hipFree(h->eig_part);
    (void)hipFree(h->vec);
    (void)hipFree(h->st);
    (void)hipFree(h->part);
    (void)hipFree(h->ndone);
    (void)hipFree(h->args_dev);
    (void)hipFree(h->flag);
    if (h->args_host) (void)hipHostFree(h->args_host);
    if (h->poll) (void)hipHostFree(h->poll);
    if (h->st_host) (void)hipHostFree(h->st_host);
    delete h;
}

sla_solve_opts default_opts() {
    sla_solve_opts o;
    o.tol = 1e-10;
    o.maxit = 1000;
    o.method = SLA_CG;
    o.precond = SLA_PRECOND_JACOBI;
    o.use_x0 = 0;
    o.graph_chunk = 0;
    o.profile = 0;
    return o;
}

sla_status check_opts(const sla_solve_opts &o) {
    if (!(o.tol >= 0.0) || o.maxit < 0) return SLA_ERR_ARG;
    if (o.method != SLA_CG && o.method != SLA_BICGSTAB) return SLA_ERR_ARG;
    if (o.precond != SLA_PRECOND_NONE && o.precond != SLA_PRECOND_JACOBI) return SLA_ERR_ARG;
    if (o.method == SLA_BICGSTAB && o.precond != SLA_PRECOND_NONE) return SLA_ERR_ARG;
    return SLA_OK;
}

// The operator a solve iterates with: A itself or the mapped A^T.  Products
// with the caller's CSR values read `cols`; the iteration kernels read `it`,
// which is either the same or the diagonal-major form (values repacked into
// the handle's buffer at the start of each system's solve).
struct Operator {
    const void *rp;
    ColArgs cols;
    int slots;
    ColArgs it;
    int it_slots;
    const RowPlan *plan;  // the products' plan for tiles past the stage
};

// Diagonal offsets that pair up around the main one: off[q] = -off[nd-1-q].
static bool mirrored(const ColArgs &c) {
    bool m = c.nd > 0;
    for (int q = 0; q < c.nd; ++q) m = m && c.off[q] == -c.off[c.nd - 1 - q];
    return m;
}

// nsys consecutive systems on the grid path (nsys <= gbatch; 1 in profile
// mode and for the BiCGStab adjoint): fill the argument blocks, run init, then
// replay/launch iteration chunks until the device reports every system done.
template <typename T, typename IT>
sla_status grid_solve_group(sla_ctx *h, const Operator &op, const T *val, const T *b, T *x,
                            SolveState *st, int nsys, const sla_solve_opts &o, hipStream_t s,
                            double *prof_ms, int64_t *prof_launches) {
    const int64_t n = h->n, nnz = h->nnz, G = h->gbatch;
    const bool cg = o.method == SLA_CG;
    const bool jac = cg && o.precond == SLA_PRECOND_JACOBI;
    const int cm = op.it.mode;
    const int slots = op.it_slots;
    const bool dmaj = cm == kColDiaMajor;
    // vector v of system j of the group: vec + (v * G + j) * n
    T *vec = reinterpret_cast<T *>(h->vec);
    auto vp = [&](int v) { return vec + (int64_t)v * G * n; };
    IterArgs<T, IT> a;
    memset(&a, 0, sizeof(a));
    a.val = dmaj ? reinterpret_cast<const T *>(h->dia) : val;
    a.rp = reinterpret_cast<const IT *>(op.rp);
    a.cols = op.it;
    // CG reads the lower diagonals through their mirrors when the pack finds
    // the values symmetric; the offsets must mirror for that
    a.cols.sym = cg && dmaj && mirrored(op.it) ? 1 : 0;
    // CG on a 3D seven-point form walks each column of planes (z-walk)
    const int zw = cg ? cg_zwalk_plan(a.cols, n, (int64_t)sizeof(T)) : 0;
    // the diagonal-major tiles: general, fast (32-bit offsets, +-1 gathers
    // across lanes) or fast with row pairs
    const int tile = dia_tile(a.cols, n, (int64_t)sizeof(T));
    a.x = x;
    a.b = b;
    a.r = vp(0);
    a.z = vp(1);
    a.q = vp(2);
    a.rh = vp(3);
    a.s = vp(4);
    a.t = vp(5);
    a.p[0] = vp(6);
    a.p[1] = vp(7);
    a.v[0] = vp(8);
    a.v[1] = vp(9);
    a.dinv = vp(10);
    a.st = st;
    a.part = h->part;
    a.ndone = h->ndone;
    a.n = n;
    a.tol = o.tol;
    a.maxit = o.maxit;
    a.use_x0 = o.use_x0;
    // one argument block per system of the group, each pointing at its own
    // data: values vstride apart, vectors n apart, state and partial sums of
    // its own.  The previous group's copy of the pinned staging blocks has
    // completed (the host waited for a chunk launched after it), so they are
    // free to rewrite.
    const int64_t vstride = dmaj ? (int64_t)op.it.nd * n : nnz;
    IterArgs<T, IT> *ah = reinterpret_cast<IterArgs<T, IT> *>(h->args_host);
    for (int j = 0; j < nsys; ++j) {
        IterArgs<T, IT> e = a;
        const int64_t o = (int64_t)j * n;
        e.val += j * vstride;
        e.x += o;
        e.b += o;
        e.dinv += o;
        e.r += o;
        e.z += o;
        e.q += o;
        e.rh += o;
        e.s += o;
        e.t += o;
        for (int k = 0; k < 2; ++k) {
            e.p[k] += o;
            e.v[k] += o;
        }
        e.st += j;
        e.part += (int64_t)j * kPartStride;
        ah[j] = e;
    }
    const IterArgs<T, IT> *ad = reinterpret_cast<const IterArgs<T, IT> *>(h->args_dev);
    HIP_TRY(hipMemcpyAsync(h->args_dev, h->args_host, sizeof(a) * nsys, hipMemcpyHostToDevice,
                           s));
    HIP_TRY(hipMemsetAsync(st, 0, sizeof(SolveState) * nsys, s));
    HIP_TRY(hipMemsetAsync(h->ndone, 0, sizeof(int32_t), s));
    if (dmaj)
        HIP_TRY(launch_dia_pack<T, IT>(a.rp, a.cols, val, nnz, reinterpret_cast<T *>(h->dia), n,
                                       nsys, st, s));
    if (jac) HIP_TRY(launch_dinv<T, IT>(reinterpret_cast<const IT *>(h->diagpos), val, nnz, vp(10),
                                        n, st, nsys, s));
    // A x0 goes to t (CG) or q (BiCGStab), which the init kernels read; CG
    // reads it always, so it is zeroed when there is no initial guess
    if (o.use_x0)
        HIP_TRY(launch_spmv<T, IT>(op.slots, a.rp, op.cols, val, nnz, x, cg ? a.t : a.q, n, n,
                                   nsys, s, op.plan));
    else if (cg)
        HIP_TRY(hipMemsetAsync(a.t, 0, sizeof(T) * n * nsys, s));
    // on an operator with a row plan (long rows) the iterations run split:
    // the fused kernels' tile walker would take those rows a wavefront each
    const bool planned_op = !dmaj && op.plan && op.plan->nitems > 0;
    const bool split = cg && planned_op;
    const bool bsplit = !cg && planned_op;
    const IT *dpos = reinterpret_cast<const IT *>(h->diagpos);
    if (split) {
        HIP_TRY(launch_cg_split_init<T, IT>(jac, ad, n, nsys, s));
        HIP_TRY(launch_spmv<T, IT>(op.slots, a.rp, op.cols, val, nnz, a.r, a.v[0], n, n, nsys, s,
                                   op.plan));
        HIP_TRY(launch_cg_split_w<T, IT>(jac, true, ad, dpos, n, nsys, 0, s));
    } else if (cg) {
        HIP_TRY(launch_cg_init<T, IT>(slots, cm, zw, jac, ad, n, nsys, s));
    } else {
        HIP_TRY(launch_bicg_init<T, IT>(cm, ad, n, nsys, s));
    }

    // split BiCGStab: half h of iteration k (0: updates, p_k -> v_k,
    // partials; 1: updates, s -> t, partials); split chunks start at even
    // iterations, so k's parity is the iteration's
    auto bicg_half = [&](hipStream_t ss, int k, int h) -> hipError_t {
        hipError_t e;
        const T *in = h ? a.s : a.p[(k + 1) & 1];
        T *out = h ? a.t : a.v[(k + 1) & 1];
        if ((e = launch_bicg_split<T, IT>(2 * h, ad, n, nsys, ss)) != hipSuccess) return e;
        if ((e = launch_spmv<T, IT>(op.slots, a.rp, op.cols, nullptr, 0, in, out, n, n, nsys, ss,
                                    op.plan, ad)) != hipSuccess)
            return e;
        return launch_bicg_split<T, IT>(2 * h + 1, ad, n, nsys, ss);
    };

    // iteration k; CG launches carry the iteration's parity
    auto one_iter = [&](hipStream_t ss, int k) -> hipError_t {
        hipError_t e;
        if (split) {
            if ((e = launch_cg_split_u<T, IT>(jac, ad, n, nsys, k & 1, ss)) != hipSuccess) return e;
            if ((e = launch_spmv<T, IT>(op.slots, a.rp, op.cols, nullptr, 0, a.r, a.v[0], n, n,
                                        nsys, ss, op.plan, ad)) != hipSuccess)
                return e;
            return launch_cg_split_w<T, IT>(jac, false, ad, dpos, n, nsys, k & 1, ss);
        }
        if (cg) return launch_cg_iter<T, IT>(slots, cm, jac, zw, tile, ad, n, nsys, k & 1, ss);
        if (bsplit) {
            if ((e = bicg_half(ss, k, 0)) != hipSuccess) return e;
            return bicg_half(ss, k, 1);
        }
        if ((e = launch_bicg_xpv<T, IT>(slots, cm, tile, ad, n, nsys, ss)) != hipSuccess) return e;
        return launch_bicg_st<T, IT>(slots, cm, tile, ad, n, nsys, ss);
    };

    if (o.profile) {
        // every iteration launched directly; each fused SpMV kernel carries a
        // pair of events that the runtime records at its start and end; the
        // stop at maxit is detected in iteration maxit (CG: its kernel;
        // BiCGStab: its second kernel), so maxit + 1 iterations are enqueued
        const int per = cg ? 1 : 2;
        const int launches = o.maxit + 1;
        const size_t need = (size_t)2 * per * (size_t)launches;
        while (h->prof_ev.size() < need) {
            hipEvent_t e;
            HIP_TRY(hipEventCreate(&e));
            h->prof_ev.push_back(e);
        }
        size_t ev = 0;
        for (int k = 0; k < launches; ++k) {
            if (split) {  // the three launches between a pair of stream events
                HIP_TRY(hipEventRecord(h->prof_ev[ev], s));
                HIP_TRY(one_iter(s, k));
                HIP_TRY(hipEventRecord(h->prof_ev[ev + 1], s));
                ev += 2;
            } else if (cg) {
                HIP_TRY(launch_cg_iter<T, IT>(slots, cm, jac, zw, tile, ad, n, 1, k & 1, s,
                                              &h->prof_ev[ev]));
                ev += 2;
            } else if (bsplit) {  // each half's three launches between stream events
                for (int hh = 0; hh < 2; ++hh) {
                    HIP_TRY(hipEventRecord(h->prof_ev[ev], s));
                    HIP_TRY(bicg_half(s, k, hh));
                    HIP_TRY(hipEventRecord(h->prof_ev[ev + 1], s));
                    ev += 2;
                }
            } else {
                HIP_TRY(launch_bicg_xpv<T, IT>(slots, cm, tile, ad, n, 1, s, &h->prof_ev[ev]));
                ev += 2;
                HIP_TRY(launch_bicg_st<T, IT>(slots, cm, tile, ad, n, 1, s, &h->prof_ev[ev]));
                ev += 2;
            }
            if ((k & 63) == 63 || k + 1 == launches) {
                HIP_TRY(launch_publish(h->ndone, h->poll_dev, s));
                HIP_TRY(hipStreamSynchronize(s));
                if (__atomic_load_n(&h->poll[0], __ATOMIC_ACQUIRE) >= nsys) break;
            }
        }
        SolveState hs;
        HIP_TRY(hipMemcpyAsync(&hs, st, sizeof(hs), hipMemcpyDeviceToHost, s));
        HIP_TRY(hipStreamSynchronize(s));
        // the first `nfused` bracketed launches did work; later ones returned
        // at entry
        int64_t active = hs.nfused;
        if ((size_t)(2 * active) > ev) active = (int64_t)(ev / 2);
        double total = 0.0;
        for (int64_t j = 0; j < active; ++j) {
            float ms = 0.f;
            HIP_TRY(hipEventElapsedTime(&ms, h->prof_ev[2 * j], h->prof_ev[2 * j + 1]));
            total += ms;
        }
        *prof_ms += total;
        *prof_launches += active;
    } else {
        // the stop is detected by the first kernel of iteration maxit, so
        // maxit + 1 iterations may be launched; CG (and split BiCGStab)
        // chunks have even length so that every chunk starts at an even
        // iteration
        // Default length: a stop leaves up to two chunks of no-op launches
        // in flight (about 2.4 us each) and every chunk boundary costs a few
        // us, so the best length grows like the square root of the iteration
        // count; the handle's previous grid solve (a forward before its
        // adjoint, the last step of a loop) predicts it.
        int chunk = o.graph_chunk < 0 ? -o.graph_chunk : o.graph_chunk;
        if (o.graph_chunk == 0)
            chunk = h->last_iters >= 1800 ? 4 * kDefaultChunk
                    : h->last_iters >= 460 ? 2 * kDefaultChunk
                                           : kDefaultChunk;
        if (chunk > o.maxit + 1) chunk = o.maxit + 1;
        if (chunk < 1) chunk = 1;
        if ((cg || bsplit) && (chunk & 1)) ++chunk;
        // direct launches when asked (graph_chunk < 0), and by default for
        // the fused iterations of large enough launches
        const bool direct =
            o.graph_chunk < 0 ||
            (o.graph_chunk == 0 && !planned_op &&
             n * nsys >= (cg ? kDirectRowsCg : kDirectRowsBicg));
        const int key = (cg ? 0 : 4) + (jac ? 1 : 0) + (op.rp != h->rp ? 2 : 0) + 8 * nsys;
        // the replayable graph of `len` iterations plus the publish of the
        // stopped count: cached per (key, len), captured on first use
        auto graph_of = [&](int len, hipGraphExec_t *out) -> hipError_t {
            for (auto &g : h->graphs)
                if (g.key == key && g.chunk == len) {
                    *out = g.exec;
                    return hipSuccess;
                }
            GraphEntry *slot = nullptr;
            for (auto &g : h->graphs)
                if (g.key == -1) {
                    slot = &g;
                    break;
                }
            if (!slot) slot = &h->graphs[h->graph_next++ % kGraphSlots];
            if (slot->exec) {
                hipError_t de = hipGraphExecDestroy(slot->exec);
                slot->exec = nullptr;
                slot->key = -1;
                if (de != hipSuccess) return de;
            }
            hipGraph_t graph = nullptr;
            hipError_t ce = hipStreamBeginCapture(h->cap, hipStreamCaptureModeThreadLocal);
            if (ce != hipSuccess) return ce;
            for (int k = 0; k < len && ce == hipSuccess; ++k) ce = one_iter(h->cap, k);
            if (ce == hipSuccess) ce = launch_publish(h->ndone, h->poll_dev, h->cap);
            hipError_t ee = hipStreamEndCapture(h->cap, &graph);
            if (ce != hipSuccess) return ce;
            if (ee != hipSuccess) return ee;
            hipError_t ie = hipGraphInstantiate(&slot->exec, graph, nullptr, nullptr, 0);
            (void)hipGraphDestroy(graph);
            if (ie != hipSuccess) return ie;
            slot->key = key;
            slot->chunk = len;
            *out = slot->exec;
            return hipSuccess;
        };
        // enough chunks to pass maxit + 1 iterations, and one more
        const int64_t need = (int64_t)o.maxit + 1;
        int64_t launched = 0;
        for (int64_t c = 0;; ++c) {
            const bool more = launched < need + chunk;
            if (more) {
                // the chunk ends with the copy of the stopped count to poll
                if (!direct) {
                    hipGraphExec_t exec = nullptr;
                    HIP_TRY(graph_of(chunk, &exec));
                    HIP_TRY(hipGraphLaunch(exec, s));
                } else {
                    for (int k = 0; k < chunk; ++k) HIP_TRY(one_iter(s, k));
                    HIP_TRY(launch_publish(h->ndone, h->poll_dev, s));
                }
                HIP_TRY(hipEventRecord(h->ev[c & 1], s));
                launched += chunk;
            }
            // chunk c - 1 has published; chunk c may have published since
            // (the count only grows), either is a state the device reached
            if (c >= 1) {
                HIP_TRY(hipEventSynchronize(h->ev[(c - 1) & 1]));
                if (__atomic_load_n(&h->poll[0], __ATOMIC_ACQUIRE) >= nsys) break;
            }
            if (!more) break;
        }
    }
    if (cg) HIP_TRY(launch_cg_lag<T>(st, a.p[0], x, n, nsys, s));
    if (o.use_x0) HIP_TRY(launch_zero_if<T>(st, x, n, nsys, s));
    return SLA_OK;
}

template <typename T, typename IT>
sla_status solve_all(sla_ctx *h, const Operator &op, const T *val, const T *b, T *x,
                     const sla_solve_opts &o, sla_solve_info *info, hipStream_t s) {
    const int64_t n = h->n, nnz = h->nnz, B = h->batch;
    const bool cg = o.method == SLA_CG;
    double prof_ms = 0.0;
    int64_t prof_launches = 0;
    const bool block_path = cg && n <= kBlockSolveMaxN && !o.profile;
    if (info) info->form = block_path ? -1 : op.it.mode;
    if (block_path) {
        BlockCgParams p;
        p.val = val;
        p.rp = op.rp;
        p.col = op.cols.col;
        p.diagpos = h->diagpos;
        p.x = x;
        p.b = b;
        p.st = h->st;
        p.n = n;
        p.nnz = nnz;
        p.tol = o.tol;
        p.maxit = o.maxit;
        p.use_x0 = o.use_x0;
        p.jac = o.precond == SLA_PRECOND_JACOBI;
        for (int64_t s0 = 0; s0 < B; s0 += 65535) {
            const int nb = (int)((B - s0) < 65535 ? (B - s0) : 65535);
            BlockCgParams q = p;
            q.val = reinterpret_cast<const T *>(val) + s0 * nnz;
            q.b = reinterpret_cast<const T *>(b) + s0 * n;
            q.x = reinterpret_cast<T *>(x) + s0 * n;
            q.st = h->st + s0;
            HIP_TRY(launch_block_cg<T, IT>(h->max_len, q, nb, s));
        }
    } else {
        const int64_t G = !o.profile ? std::min(h->gbatch, B) : 1;
        for (int64_t s0 = 0; s0 < B; s0 += G) {
            const int nsys = (int)std::min(G, B - s0);
            sla_status r = grid_solve_group<T, IT>(h, op, val + s0 * nnz, b + s0 * n, x + s0 * n,
                                                   h->st + s0, nsys, o, s, &prof_ms,
                                                   &prof_launches);
            if (r != SLA_OK) return r;
        }
    }
    HIP_TRY(hipMemcpyAsync(h->st_host, h->st, sizeof(SolveState) * B, hipMemcpyDeviceToHost, s));
    HIP_TRY(hipStreamSynchronize(s));
    int worst_err = 0, worst_pos = 0;
    bool sym = !block_path && cg && op.it.mode == kColDiaMajor && mirrored(op.it);
    int32_t most = 0;
    for (int64_t sys = 0; sys < B; ++sys) {
        const SolveState &ss = h->st_host[sys];
        const int stc = ss.status;
        sym = sym && !ss.asym;
        most = std::max(most, ss.iter);
        if (stc < 0 && stc < worst_err) worst_err = stc;
        if (stc > worst_pos) worst_pos = stc;
        if (info) {
            if (info->iters) info->iters[sys] = ss.iter;
            if (info->spmv) info->spmv[sys] = ss.spmv;
            if (info->status) info->status[sys] = stc;
            if (info->relres) info->relres[sys] = ss.bb > 0.0 ? sqrt(ss.rr) / sqrt(ss.bb) : 0.0;
        }
    }
    if (!block_path) h->last_iters = most;
    if (info) {
        info->kernel_ms = prof_ms;
        info->kernel_launches = prof_launches;
        if (sym) info->form = 4;
    }
    return (sla_status)(worst_err < 0 ? worst_err : worst_pos);
}

template <typename T, typename IT>
sla_status adjoint_all(sla_ctx *h, const T *val, const T *x, const T *gx, T *gval, T *gb,
                       const sla_solve_opts &o, sla_solve_info *info, hipStream_t s) {
    const int64_t n = h->n, nnz = h->nnz, B = h->batch;
    sla_solve_opts oo = o;
    oo.use_x0 = 0;
    sla_status st;
    if (o.method == SLA_CG) {
        Operator op{h->rp, h->ca, h->slots, h->ia, h->it_slots, &h->plan};
        st = solve_all<T, IT>(h, op, val, gx, gb, oo, info, s);
    } else {
        // A^T with its values put in A^T's order, one system at a time into
        // the handle's buffer
        Operator op{h->rp_t, h->ca_t, h->slots_t, h->ia_t, h->it_slots_t, &h->plan_t};
        const int64_t B0 = h->batch;
        st = SLA_OK;
        std::vector<int32_t> it(B0), mv(B0), stc(B0);
        std::vector<double> rr(B0);
        double kms = 0.0;
        int64_t kl = 0;
        h->batch = 1;
        for (int64_t sys = 0; sys < B0; ++sys) {
            hipError_t e = launch_scatter<T>(h->pinv, val + sys * nnz,
                                             reinterpret_cast<T *>(h->val_t), nnz, s);
            if (e != hipSuccess) {
                h->batch = B0;
                g_last_error = e;
                return SLA_ERR_DEVICE;
            }
            sla_solve_info one{};
            one.iters = &it[sys];
            one.spmv = &mv[sys];
            one.relres = &rr[sys];
            one.status = &stc[sys];
            sla_status r = solve_all<T, IT>(h, op, reinterpret_cast<const T *>(h->val_t), gx + sys * n,
                                            gb + sys * n, oo, &one, s);
            kms += one.kernel_ms;
            kl += one.kernel_launches;
            if (info) info->form = one.form;
            if (r < 0 && (st >= 0 || r < st)) st = r;
            if (r > 0 && st >= 0 && r > st) st = r;
            if (r == SLA_ERR_DEVICE) break;
        }
        h->batch = B0;
        if (info) {
            for (int64_t sys = 0; sys < B0; ++sys) {
                if (info->iters) info->iters[sys] = it[sys];
                if (info->spmv) info->spmv[sys] = mv[sys];
                if (info->relres) info->relres[sys] = rr[sys];
                if (info->status) info->status[sys] = stc[sys];
            }
            info->kernel_ms = kms;
            info->kernel_launches = kl;
        }
    }
    if (st == SLA_ERR_DEVICE) return st;
    for (int64_t s0 = 0; s0 < B; s0 += 65535) {
        const int nb = (int)((B - s0) < 65535 ? (B - s0) : 65535);
        HIP_TRY(launch_grad<T, IT>(reinterpret_cast<const IT *>(h->rp), h->ca, gb + s0 * n,
                                   x + s0 * n, gval + s0 * nnz, n, nnz, nb, true, s, &h->plan));
    }
    HIP_TRY(hipStreamSynchronize(s));
    return st;
}

// Compact columns for the pattern (rp, col), longest row max_len, when
// every entry fits; rowidx (the row of every entry) serves patterns with
// long rows, which are checked entry by entry.
template <typename IT>
hipError_t build_col16(sla_ctx *h, const IT *rp, const int32_t *col, int32_t max_len,
                       const int32_t *rowidx, int16_t **out, hipStream_t s) {
    int32_t fits = 0;
    const int32_t *ri = setup_entrywise(max_len, h->nnz) ? rowidx : nullptr;
    if (setup_entrywise(max_len, h->nnz) && !ri) return hipSuccess;  // no row index: keep int32
    hipError_t e = setup_col16<IT>(rp, col, h->n, h->nnz, ri, nullptr, h->flag, &fits, s);
    if (e != hipSuccess || !fits) return e;
    if ((e = dmalloc(h, out, sizeof(int16_t) * h->nnz)) != hipSuccess) return e;
    return setup_col16<IT>(rp, col, h->n, h->nnz, ri, *out, h->flag, &fits, s);
}

// The set-up's temporaries: one allocation for the lifetime of sla_create.
struct SetupMem {
    void *base = nullptr;
    SetupScratch scr;
    ~SetupMem() { (void)hipFree(base); }
};

// Diagonal masks for the pattern (rp, col) when its entries lie on at most
// kMaxDiags diagonals and no row holds more than 8 of them; fills `ca`.
template <typename IT>
hipError_t build_diag(sla_ctx *h, const IT *rp, const int32_t *col, int32_t max_len,
                      int32_t *dlt_dev, uint16_t **msk, ColArgs &ca, hipStream_t s) {
    if (max_len > 8) return hipSuccess;
    int32_t dlt[kMaxDiags], nd = 0;
    hipError_t e = setup_diag<IT>(rp, col, h->n, dlt_dev, h->flag, dlt, &nd, s);
    if (e != hipSuccess || nd == 0) return e;
    if ((e = hipMemcpyAsync(dlt_dev, dlt, sizeof(dlt), hipMemcpyHostToDevice, s)) != hipSuccess)
        return e;
    if ((e = dmalloc(h, msk, sizeof(uint16_t) * h->n)) != hipSuccess) return e;
    if ((e = setup_diag_masks<IT>(rp, col, h->n, dlt_dev, nd, *msk, s)) != hipSuccess) return e;
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;  // dlt is a host buffer
    int nneg = 0;
    while (nneg < nd && dlt[nneg] < 0) ++nneg;
    ca.msk = *msk;
    ca.dlt = dlt_dev;
    ca.nneg = nneg;
    ca.nd = nd;
    for (int q = 0; q < nd && q < kMaxDiaMajor; ++q) ca.off[q] = dlt[q];
    ca.mode = kColDiag;
    return hipSuccess;
}

// The row plan of a pattern whose row pointers are rp_dev (see RowPlan):
// the tiles whose entries exceed the tile walker's stage or that hold a row
// longer than its slots (the products' gather slots per row).  Built on the
// host from a copy of the row pointers when the longest row exceeds
// kCap / kTileRows (below that no tile needs it; the walker's slots cover
// at least 4 entries), kept only if some tile needs it.  which: 0 for A, 1
// for A^T; partial sums for up to 65535 systems (one launch's batch).
template <typename T, typename IT>
hipError_t build_plan(sla_ctx *h, int which, const IT *rp_dev, const int32_t *col,
                      int32_t max_len, int slots, RowPlan &pl, hipStream_t s) {
    pl = RowPlan();
    if ((int64_t)max_len * kTileRows <= kCap && max_len <= slots) return hipSuccess;
    const int64_t n = h->n;
    std::vector<IT> rp((size_t)n + 1);
    hipError_t e = hipMemcpyAsync(rp.data(), rp_dev, sizeof(IT) * (n + 1), hipMemcpyDeviceToHost, s);
    if (e != hipSuccess || (e = hipStreamSynchronize(s)) != hipSuccess) return e;
    std::vector<PlanItem> items;
    std::vector<PlanFin> fin;
    std::vector<uint8_t> tiles((size_t)tiles_of(n), 0);
    int32_t nslots = 0;
    int64_t ntiles_planned = 0;
    for (int64_t t = 0; t < tiles_of(n); ++t) {
        const int64_t a = t * kTileRows, b = std::min<int64_t>(a + kTileRows, n);
        int64_t longest = 0;
        for (int64_t r = a; r < b; ++r) longest = std::max<int64_t>(longest, rp[r + 1] - rp[r]);
        if ((int64_t)(rp[b] - rp[a]) <= kCap && longest <= slots) continue;  // the walker's
        tiles[(size_t)t] = 1;
        ++ntiles_planned;
        for (int64_t r = a; r < b;) {
            const int64_t len = (int64_t)(rp[r + 1] - rp[r]);
            if (len > kShortRow) {  // a long row: chunks of kPlanCap entries
                const int64_t nch = (len + kPlanCap - 1) / kPlanCap;
                if (nch > 1) fin.push_back(PlanFin{(int32_t)r, nslots, (int32_t)nch, 0});
                for (int64_t c = 0; c < nch; ++c) {
                    const int64_t e0 = (int64_t)rp[r] + c * kPlanCap;
                    items.push_back(PlanItem{(int32_t)r, (int32_t)(r + 1),
                                             nch > 1 ? nslots + (int32_t)c : -1, 1, e0,
                                             std::min<int64_t>(e0 + kPlanCap, (int64_t)rp[r + 1])});
                }
                if (nch > 1) nslots += (int32_t)nch;
                ++r;
                continue;
            }
            // a short block: consecutive short rows while the run fits kPlanCap
            const int64_t r0 = r;
            while (r < b && (int64_t)(rp[r + 1] - rp[r]) <= kShortRow &&
                   (int64_t)(rp[r + 1] - rp[r0]) <= kPlanCap)
                ++r;
            items.push_back(PlanItem{(int32_t)r0, (int32_t)r, -1, 0, (int64_t)rp[r0],
                                     (int64_t)rp[r]});
        }
    }
    if (items.empty()) return hipSuccess;
    void **mem = h->plan_mem[which];
    if ((e = dmalloc(h, (uint8_t **)&mem[3], tiles.size())) != hipSuccess) return e;
    if ((e = hipMemcpyAsync(mem[3], tiles.data(), tiles.size(), hipMemcpyHostToDevice, s)) !=
        hipSuccess)
        return e;
    if ((e = dmalloc(h, (PlanItem **)&mem[0], sizeof(PlanItem) * items.size())) != hipSuccess)
        return e;
    if ((e = hipMemcpyAsync(mem[0], items.data(), sizeof(PlanItem) * items.size(),
                            hipMemcpyHostToDevice, s)) != hipSuccess)
        return e;
    if (!fin.empty()) {
        if ((e = dmalloc(h, (PlanFin **)&mem[1], sizeof(PlanFin) * fin.size())) != hipSuccess)
            return e;
        if ((e = hipMemcpyAsync(mem[1], fin.data(), sizeof(PlanFin) * fin.size(),
                                hipMemcpyHostToDevice, s)) != hipSuccess)
            return e;
        const int64_t sys = std::min<int64_t>(h->batch, 65535);
        if ((e = dmalloc(h, (T **)&mem[2], sizeof(T) * (size_t)nslots * sys)) != hipSuccess)
            return e;
    }
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;  // items and fin are host buffers
    pl.tiles = reinterpret_cast<const uint8_t *>(mem[3]);
    pl.all_tiles = ntiles_planned == (int64_t)tiles.size();
    pl.items = reinterpret_cast<const PlanItem *>(mem[0]);
    pl.nitems = (int32_t)items.size();
    pl.fin = reinterpret_cast<const PlanFin *>(mem[1]);
    pl.nfin = (int32_t)fin.size();
    pl.nslots = nslots;
    pl.col = col;
    pl.part = mem[2];
    return hipSuccess;
}

template <typename T, typename IT>
sla_status create_typed(sla_ctx *h, int32_t flags, hipStream_t s) {
    const bool build_t = (flags & SLA_CREATE_TRANSPOSE) != 0;
    const bool compact = (flags & SLA_CREATE_WIDE_COLUMNS) == 0;
    const bool dmajor = compact && (flags & SLA_CREATE_CSR_VALUES) == 0;
    const int64_t n = h->n, nnz = h->nnz;
    const IT *rp = reinterpret_cast<const IT *>(h->rp);
    HIP_TRY(dmalloc(h, &h->diagpos, sizeof(IT) * n));
    HIP_TRY(dmalloc(h, &h->flag, sizeof(int32_t)));
    int32_t bad = 0;
    HIP_TRY(setup_check_rowptr<IT>(rp, n, nnz, h->flag, &bad, s));
    if (bad) return SLA_ERR_PATTERN;  // columns not read
    int32_t maxlen = 0;
    HIP_TRY(setup_max_row<IT>(rp, n, h->flag, &maxlen, s));
    // the row of every entry serves the entry-by-entry checks of patterns
    // with long rows and the transpose; one allocation holds it and the
    // transpose's temporaries until the end of the set-up
    const bool entrywise = setup_entrywise(maxlen, nnz);
    SetupMem tmp;
    if (entrywise || build_t) {
        HIP_TRY(hipMalloc(&tmp.base, (size_t)setup_scratch_bytes(nnz, true, build_t)));
        setup_scratch_carve(tmp.base, nnz, true, build_t, &tmp.scr);
        HIP_TRY(setup_row_index<IT>(rp, n, nnz, tmp.scr.rowidx, tmp.scr.tot, s));
    }
    HIP_TRY(setup_check_cols<IT>(rp, h->col, n, nnz, entrywise ? tmp.scr.rowidx : nullptr,
                                 reinterpret_cast<IT *>(h->diagpos), h->flag, &bad, s));
    if (bad) return SLA_ERR_PATTERN;
    h->slots = slots_for(maxlen);
    h->max_len = maxlen;
    h->slots_t = h->slots;
    HIP_TRY((build_plan<T, IT>(h, 0, rp, h->col, maxlen, h->slots, h->plan, s)));
    if (build_t) {
        HIP_TRY(dmalloc(h, &h->rp_t, sizeof(IT) * (n + 1)));
        HIP_TRY(dmalloc(h, &h->col_t, sizeof(int32_t) * nnz));
        HIP_TRY(dmalloc(h, &h->perm, sizeof(int32_t) * nnz));
        HIP_TRY(dmalloc(h, &h->pinv, sizeof(int32_t) * nnz));
        HIP_TRY(dmalloc(h, &h->val_t, sizeof(T) * nnz));
        HIP_TRY(setup_transpose<IT>(rp, h->col, n, nnz, reinterpret_cast<IT *>(h->rp_t), h->col_t,
                                    h->perm, h->pinv, tmp.scr, s));
        h->has_t = true;
        HIP_TRY(setup_max_row<IT>(reinterpret_cast<const IT *>(h->rp_t), n, h->flag, &maxlen, s));
        h->slots_t = slots_for(maxlen);
        h->ca_t.col = h->col_t;
        HIP_TRY((build_plan<T, IT>(h, 1, reinterpret_cast<const IT *>(h->rp_t), h->col_t, maxlen,
                                   h->slots_t, h->plan_t, s)));
        if (compact) {
            const IT *rpt = reinterpret_cast<const IT *>(h->rp_t);
            HIP_TRY(build_col16<IT>(h, rpt, h->col_t, maxlen, tmp.scr.rowidx_t, &h->col16_t, s));
            h->ca_t.col16 = h->col16_t;
            if (h->col16_t) h->ca_t.mode = kColTile16;
            HIP_TRY(dmalloc(h, &h->dlt, sizeof(int32_t) * 2 * kMaxDiags));
            HIP_TRY(build_diag<IT>(h, rpt, h->col_t, maxlen, h->dlt + kMaxDiags, &h->msk_t,
                                   h->ca_t, s));
        }
    }
    h->ca.col = h->col;
    if (compact) {
        HIP_TRY(build_col16<IT>(h, rp, h->col, h->max_len, tmp.scr.rowidx, &h->col16, s));
        h->ca.col16 = h->col16;
        if (h->col16) h->ca.mode = kColTile16;
        if (!h->dlt) HIP_TRY(dmalloc(h, &h->dlt, sizeof(int32_t) * 2 * kMaxDiags));
        HIP_TRY(build_diag<IT>(h, rp, h->col, h->max_len, h->dlt, &h->msk, h->ca, s));
        if (h->ca.mode != kColDiag && h->ca_t.mode != kColDiag) {  // the table went unused
            HIP_TRY(hipFree(h->dlt));
            h->dlt = nullptr;
            h->ws_bytes -= (int64_t)sizeof(int32_t) * 2 * kMaxDiags;
        }
    }
    // the two-pass A^T products of the per-entry column forms write their
    // terms tile by tile of A^T in A's entry order (setup_buckets)
    if (h->has_t && h->ca.mode != kColDiag) {
        HIP_TRY(dmalloc(h, &h->bpos, sizeof(int32_t) * nnz));
        HIP_TRY(dmalloc(h, &h->lidx, sizeof(uint16_t) * nnz));
        HIP_TRY(setup_buckets<IT>(reinterpret_cast<const IT *>(h->rp_t), h->perm, h->plan_t, n,
                                  nnz, h->bpos, h->lidx, s));
    }
    // The iterations read diagonal-major values for patterns on 3, 5 or 7
    // diagonals with the main one in the middle (nearest-neighbour stencils
    // in 1, 2 and 3 dimensions) whose padding -- the slots of boundary rows
    // that lack a diagonal -- stays within a quarter of the stored entries;
    // one copy per system of a launch group is kept.
    h->ia = h->ca;
    h->it_slots = h->slots;
    h->ia_t = h->ca_t;
    h->it_slots_t = h->slots_t;
    int nd = 0;
    if (dmajor) {
        auto fits = [&](const ColArgs &c) {
            return c.mode == kColDiag && (c.nd == 3 || c.nd == 5 || c.nd == 7) &&
                   c.nneg == c.nd / 2 && (int64_t)c.nd * n <= nnz + nnz / 4;
        };
        if (fits(h->ca)) {
            h->ia.mode = kColDiaMajor;
            h->it_slots = nd = h->ca.nd;
        }
        if (h->has_t && fits(h->ca_t)) {
            h->ia_t.mode = kColDiaMajor;
            h->it_slots_t = h->ca_t.nd;
            nd = std::max(nd, (int)h->ca_t.nd);
        }
    }
    // CG and BiCGStab on a batch of systems too large for the one-workgroup
    // solver advance up to gbatch of them per grid launch
    if (h->batch > 1 && n > kBlockSolveMaxN)
        h->gbatch = std::max<int64_t>(1, std::min<int64_t>({h->batch, 65535, kGroupRows / n}));
    if (nd) HIP_TRY(dmalloc(h, &h->dia, sizeof(T) * (size_t)nd * n * h->gbatch));
    HIP_TRY(dmalloc(h, &h->vec, sizeof(T) * (size_t)kNumVec * n * h->gbatch));
    HIP_TRY(dmalloc(h, &h->st, sizeof(SolveState) * h->batch));
    HIP_TRY(dmalloc(h, &h->part, sizeof(double) * kPartStride * h->gbatch));
    HIP_TRY(dmalloc(h, &h->ndone, sizeof(int32_t)));
    HIP_TRY(dmalloc(h, &h->args_dev, sizeof(IterArgs<T, IT>) * h->gbatch));
    HIP_TRY(hipHostMalloc(&h->args_host, sizeof(IterArgs<T, IT>) * h->gbatch,
                          hipHostMallocDefault));
    HIP_TRY(hipHostMalloc((void **)&h->poll, 2 * sizeof(int32_t),
                          hipHostMallocMapped | hipHostMallocCoherent));
    HIP_TRY(hipHostGetDevicePointer((void **)&h->poll_dev, h->poll, 0));
    HIP_TRY(hipHostMalloc((void **)&h->st_host, sizeof(SolveState) * h->batch, hipHostMallocDefault));
    HIP_TRY(hipMemsetAsync(h->st, 0, sizeof(SolveState) * h->batch, s));
    HIP_TRY(hipMemsetAsync(h->part, 0, sizeof(double) * kPartStride * h->gbatch, s));
    HIP_TRY(hipStreamCreateWithFlags(&h->cap, hipStreamNonBlocking));
    HIP_TRY(hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking));
    HIP_TRY(hipEventCreateWithFlags(&h->fork, hipEventDisableTiming));
    HIP_TRY(hipEventCreateWithFlags(&h->join, hipEventDisableTiming));
    HIP_TRY(hipEventCreateWithFlags(&h->ev[0], hipEventDisableTiming));
    HIP_TRY(hipEventCreateWithFlags(&h->ev[1], hipEventDisableTiming));
    HIP_TRY(hipStreamSynchronize(s));
    return SLA_OK;
}

template <typename F>
sla_status dispatch(const sla_ctx *h, F &&f) {
    if (h->dtype == SLA_F64) {
        if (h->itype == SLA_I64) return f((double *)nullptr, (int64_t *)nullptr);
        return f((double *)nullptr, (int32_t *)nullptr);
    }
    if (h->itype == SLA_I64) return f((float *)nullptr, (int64_t *)nullptr);
    return f((float *)nullptr, (int32_t *)nullptr);
}


// ------------------------------------------------------------- eigensolver

// Eigen-decomposition of a small dense symmetric matrix by cyclic Jacobi
// rotations (Golub & Van Loan, Matrix Computations, the symmetric Jacobi
// method): each rotation zeroes one off-diagonal pair; sweeps repeat until
// the off-diagonal part is negligible.  a [m][m] row-major is overwritten;
// column q of Q is the eigenvector of evals[q].
void jacobi_eig(std::vector<double> &a, int m, std::vector<double> &evals,
                std::vector<double> &Q) {
    Q.assign((size_t)m * m, 0.0);
    for (int i = 0; i < m; ++i) Q[(size_t)i * m + i] = 1.0;
    double total = 0.0;
    for (double x : a) total += x * x;
    for (int sweep = 0; sweep < 100; ++sweep) {
        double off = 0.0;
        for (int p = 0; p < m; ++p)
            for (int q = p + 1; q < m; ++q) off += 2.0 * a[(size_t)p * m + q] * a[(size_t)p * m + q];
        if (off <= 1e-32 * total || off == 0.0) break;
        for (int p = 0; p < m; ++p)
            for (int q = p + 1; q < m; ++q) {
                const double apq = a[(size_t)p * m + q];
                if (apq == 0.0) continue;
                const double app = a[(size_t)p * m + p], aqq = a[(size_t)q * m + q];
                const double theta = (aqq - app) / (2.0 * apq);
                const double t = (theta >= 0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
                const double c = 1.0 / sqrt(t * t + 1.0), sn = t * c;
                for (int r = 0; r < m; ++r) {  // columns p, q
                    const double arp = a[(size_t)r * m + p], arq = a[(size_t)r * m + q];
                    a[(size_t)r * m + p] = c * arp - sn * arq;
                    a[(size_t)r * m + q] = sn * arp + c * arq;
                }
                for (int r = 0; r < m; ++r) {  // rows p, q
                    const double apr = a[(size_t)p * m + r], aqr = a[(size_t)q * m + r];
                    a[(size_t)p * m + r] = c * apr - sn * aqr;
                    a[(size_t)q * m + r] = sn * apr + c * aqr;
                }
                for (int r = 0; r < m; ++r) {
                    const double qrp = Q[(size_t)r * m + p], qrq = Q[(size_t)r * m + q];
                    Q[(size_t)r * m + p] = c * qrp - sn * qrq;
                    Q[(size_t)r * m + q] = sn * qrp + c * qrq;
                }
            }
    }
    evals.resize(m);
    for (int i = 0; i < m; ++i) evals[i] = a[(size_t)i * m + i];
}

// A fixed pseudo-random start vector in [-1, 1) (the SplitMix64 output
// function of the index), so every run starts from the same vector.
inline double start_entry(uint64_t i) {
    uint64_t z = i + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}

// Views of the handle's eigensolver buffers for one call.
struct EigWork {
    void *V = nullptr;       // [m + 1][n] basis
    double *sc = nullptr;    // alpha [m], beta [m], coef [m + 1], S [m * k], norm [1]
    double *part = nullptr;  // partial sums
};

constexpr int64_t kEigPartBlocks = 256;  // partial sums per basis vector

// The handle's basis for m Lanczos vectors and k eigenpairs: kept from the
// largest call so far, reallocated (once per larger request) when too small.
template <typename T>
hipError_t eig_buffers(sla_ctx *h, int m, int k, EigWork *w) {
    if (m > h->eig_m || k > h->eig_k) {
        const int mm = m > h->eig_m ? m : h->eig_m;
        const int kk = k > h->eig_k ? k : h->eig_k;
        (void)hipFree(h->eig_V);
        (void)hipFree(h->eig_sc);
        (void)hipFree(h->eig_part);
        h->eig_V = nullptr;
        h->eig_sc = h->eig_part = nullptr;
        h->ws_bytes -= h->eig_bytes;
        h->eig_bytes = 0;
        h->eig_m = h->eig_k = 0;
        const int64_t bytes = (int64_t)sizeof(T) * (mm + 1) * h->n +
                              (int64_t)sizeof(double) * (3 * mm + 2 + mm * kk) +
                              (int64_t)sizeof(double) * kEigPartBlocks * (mm + 1);
        hipError_t e;
        if ((e = hipMalloc(&h->eig_V, sizeof(T) * (size_t)(mm + 1) * h->n)) != hipSuccess) return e;
        if ((e = hipMalloc((void **)&h->eig_sc, sizeof(double) * (size_t)(3 * mm + 2 + mm * kk))) !=
            hipSuccess)
            return e;
        if ((e = hipMalloc((void **)&h->eig_part,
                           sizeof(double) * (size_t)kEigPartBlocks * (mm + 1))) != hipSuccess)
            return e;
        h->eig_m = mm;
        h->eig_k = kk;
        h->eig_bytes = bytes;
        h->ws_bytes += bytes;
    }
    w->V = h->eig_V;
    w->sc = h->eig_sc;
    w->part = h->eig_part;
    return hipSuccess;
}

// Lanczos with full reorthogonalisation (two Gram-Schmidt passes) and
// explicit restarts from the sum of the wanted Ritz vectors, for one system.
template <typename T, typename IT>
sla_status eigsh_one(sla_ctx *h, const T *val, const sla_eig_opts &o, int m, double *evals,
                     T *X, int32_t *restarts, EigWork &wk, hipStream_t s) {
    const int64_t n = h->n;
    const int k = o.k;
    T *V = reinterpret_cast<T *>(wk.V);
    double *alpha = wk.sc, *beta = alpha + m, *coef = beta + m, *S = coef + m + 1,
           *nrm = S + (size_t)m * k;
    const IT *rp = reinterpret_cast<const IT *>(h->rp);
    // start vector
    {
        std::vector<T> v0((size_t)n);
        for (int64_t i = 0; i < n; ++i) v0[(size_t)i] = (T)start_entry((uint64_t)i);
        HIP_TRY(hipMemcpyAsync(V, v0.data(), sizeof(T) * n, hipMemcpyHostToDevice, s));
        HIP_TRY(launch_eig_dots<T>(V, 1, V, n, wk.part, nrm, true, s));
        HIP_TRY(launch_eig_scale<T>(V, V, nrm, 1e-200, n, s));
        HIP_TRY(hipStreamSynchronize(s));  // v0 is a host buffer
    }
    std::vector<double> ha((size_t)m), hb((size_t)m), th, Q, Tm, Sh((size_t)m * k);
    sla_status status = SLA_NOT_CONVERGED;
    int r = 0;
    for (;; ++r) {
        for (int j = 0; j < m; ++j) {
            T *vj = V + (size_t)j * n;
            T *w = V + (size_t)(j + 1) * n;
            HIP_TRY(launch_spmv<T, IT>(h->slots, rp, h->ca, val, 0, vj, w, n, 0, 1, s, &h->plan));
            if (j > 0) HIP_TRY(launch_eig_update<T>(w, vj - n, 1, beta + j - 1, n, s));
            HIP_TRY(launch_eig_dots<T>(vj, 1, w, n, wk.part, alpha + j, false, s));
            HIP_TRY(launch_eig_update<T>(w, vj, 1, alpha + j, n, s));
            for (int pass = 0; pass < 2; ++pass) {
                HIP_TRY(launch_eig_dots<T>(V, j + 1, w, n, wk.part, coef, false, s));
                HIP_TRY(launch_eig_update<T>(w, V, j + 1, coef, n, s));
            }
            HIP_TRY(launch_eig_dots<T>(w, 1, w, n, wk.part, beta + j, true, s));
            HIP_TRY(launch_eig_scale<T>(w, w, beta + j, 1e-200, n, s));
        }
        HIP_TRY(hipMemcpyAsync(ha.data(), alpha, sizeof(double) * m, hipMemcpyDeviceToHost, s));
        HIP_TRY(hipMemcpyAsync(hb.data(), beta, sizeof(double) * m, hipMemcpyDeviceToHost, s));
        HIP_TRY(hipStreamSynchronize(s));
        // the basis stops at an invariant subspace (beta negligible)
        double scale = 0.0;
        for (int j = 0; j < m; ++j) scale = fmax(scale, fabs(ha[j]) + fabs(hb[j]));
        int me = m;
        for (int j = 0; j < m; ++j)
            if (!(hb[j] > 1e-12 * scale)) {
                me = j + 1;
                break;
            }
        Tm.assign((size_t)me * me, 0.0);
        for (int j = 0; j < me; ++j) {
            Tm[(size_t)j * me + j] = ha[j];
            if (j + 1 < me) Tm[(size_t)j * me + j + 1] = Tm[(size_t)(j + 1) * me + j] = hb[j];
        }
        jacobi_eig(Tm, me, th, Q);
        std::vector<int> idx(me);
        for (int j = 0; j < me; ++j) idx[j] = j;
        std::sort(idx.begin(), idx.end(), [&](int a, int b) {
            return o.largest ? th[a] > th[b] : th[a] < th[b];
        });
        const int kk = k < me ? k : me;
        double tmax = 0.0;
        for (int q = 0; q < kk; ++q) tmax = fmax(tmax, fabs(th[idx[q]]));
        bool ok = kk == k;
        const double bl = me < m ? 0.0 : hb[me - 1];
        for (int q = 0; q < kk; ++q) {
            evals[q] = th[idx[q]];
            const double res = bl * fabs(Q[(size_t)(me - 1) * me + idx[q]]);
            ok = ok && res <= o.tol * (tmax > 0.0 ? tmax : 1.0);
        }
        for (int q = kk; q < k; ++q) evals[q] = NAN;
        std::fill(Sh.begin(), Sh.end(), 0.0);
        for (int j = 0; j < me; ++j)
            for (int q = 0; q < kk; ++q) Sh[(size_t)j * k + q] = Q[(size_t)j * me + idx[q]];
        HIP_TRY(hipMemcpyAsync(S, Sh.data(), sizeof(double) * me * k, hipMemcpyHostToDevice, s));
        HIP_TRY(launch_eig_combine<T>(X, V, me, k, S, n, s));
        HIP_TRY(hipStreamSynchronize(s));  // Sh is reused
        if (ok) {
            status = SLA_OK;
            break;
        }
        if (r >= o.max_restarts) break;
        // restart from the sum of the wanted Ritz vectors
        std::vector<double> ones((size_t)k, -1.0);
        HIP_TRY(hipMemcpyAsync(coef, ones.data(), sizeof(double) * k, hipMemcpyHostToDevice, s));
        HIP_TRY(hipMemsetAsync(V, 0, sizeof(T) * n, s));
        HIP_TRY(launch_eig_update<T>(V, X, k, coef, n, s));  // V_0 = sum_q X_q
        HIP_TRY(launch_eig_dots<T>(V, 1, V, n, wk.part, nrm, true, s));
        HIP_TRY(launch_eig_scale<T>(V, V, nrm, 1e-200, n, s));
        HIP_TRY(hipStreamSynchronize(s));  // `ones` is a host buffer
    }
    if (restarts) *restarts = r;
    return status;
}

}  // namespace

namespace {

// The backward pass and A^T products of the per-entry column forms go in two
// passes (A's rows write the terms v_k g_i to the handle's buffer at bpos,
// then A^T's rows are summed, the terms of a run put back in A^T's order in
// LDS) one system at a time, for single systems and for patterns of at least
// this many entries; smaller batches read A^T's values through the transpose
// map in one launch for all.  Both ways give the same bits.  On power-law
// graphs the A^T product alone took 74.9 / 224.7 / 440.4 us in two passes at
// 2^20 / 2^21 / 2^22 rows, against 332.0 / 669.3 us through the map at
// 2^21 / 2^22 and 112.4 us at 2^20 when the first pass wrote every term
// straight to its place in A^T's order.
constexpr int64_t kScatterMinEntries = (int64_t)1 << 20;

bool two_pass(const sla_ctx *h, int batch) {
    return h->ca.mode != kColDiag && h->bpos && (batch == 1 || h->nnz >= kScatterMinEntries);
}

// For `batch` systems: grad_x = A^T g (when gx is not null) and grad_values
// = g_i x_j on the pattern (when gv is not null).
template <typename T, typename IT>
hipError_t product_backward(sla_ctx *h, const T *v, const T *x, const T *g, T *gx, T *gv,
                            int batch, hipStream_t s) {
    const IT *rp = reinterpret_cast<const IT *>(h->rp);
    const IT *rpt = reinterpret_cast<const IT *>(h->rp_t);
    const int64_t n = h->n, nnz = h->nnz;
    if (h->ca.mode == kColDiag)  // both outputs from one pass over A's rows
        return launch_diag_vjp<T, IT>(rp, h->ca, v, nnz, g, x, gx, gv, n, nnz, batch, false, s);
    if (gx && two_pass(h, batch)) {
        T *c = reinterpret_cast<T *>(h->val_t);
        // the gradient pass (random x gathers) runs on a side stream beside
        // the A^T passes (streaming reads, runs of writes)
        if (gv) {
            hipError_t e = hipEventRecord(h->fork, s);
            if (e == hipSuccess) e = hipStreamWaitEvent(h->side, h->fork, 0);
            if (e == hipSuccess)
                e = launch_grad<T, IT>(rp, h->ca, g, x, gv, n, nnz, batch, false, h->side, &h->plan);
            if (e == hipSuccess) e = hipEventRecord(h->join, h->side);
            if (e != hipSuccess) return e;
        }
        for (int sys = 0; sys < batch; ++sys) {
            hipError_t e = launch_terms_t<T, IT>(rp, h->ca, g + sys * n, v + sys * nnz, h->bpos, c,
                                                 n, nnz, 1, s, &h->plan);
            if (e == hipSuccess)
                e = launch_rowsum<T, IT>(rpt, c, nnz, nullptr, nullptr, nullptr, gx + sys * n, n,
                                         1, s, &h->plan_t, h->lidx);
            if (e != hipSuccess) return e;
        }
        if (gv) return hipStreamWaitEvent(s, h->join, 0);
        return hipSuccess;
    } else if (gx) {
        hipError_t e = launch_rowsum<T, IT>(rpt, v, nnz, h->perm, h->col_t, g, gx, n, batch, s,
                                            &h->plan_t);
        if (e != hipSuccess) return e;
    }
    if (gv) return launch_grad<T, IT>(rp, h->ca, g, x, gv, n, nnz, batch, false, s, &h->plan);
    return hipSuccess;
}

}  // namespace

extern "C" {

sla_status sla_create(sla_handle *out, int64_t n, int64_t nnz, int64_t batch, int32_t dtype,
                      int32_t row_ptr_type, const void *d_row_ptr, const int32_t *d_col,
                      int32_t flags, void *stream) {
    if (!out) return SLA_ERR_ARG;
    *out = nullptr;
    if (n < 1 || n >= ((int64_t)1 << 31) || nnz < n || batch < 1) return SLA_ERR_ARG;
    if (dtype != SLA_F32 && dtype != SLA_F64) return SLA_ERR_ARG;
    if (row_ptr_type != SLA_I32 && row_ptr_type != SLA_I64) return SLA_ERR_ARG;
    if (row_ptr_type == SLA_I32 && nnz >= ((int64_t)1 << 31)) return SLA_ERR_ARG;
    if (flags & ~(SLA_CREATE_TRANSPOSE | SLA_CREATE_WIDE_COLUMNS | SLA_CREATE_CSR_VALUES))
        return SLA_ERR_ARG;
    if ((flags & SLA_CREATE_TRANSPOSE) && nnz >= ((int64_t)1 << 31)) return SLA_ERR_ARG;
    if (!d_row_ptr || !d_col) return SLA_ERR_ARG;
    sla_ctx *h = new (std::nothrow) sla_ctx();
    if (!h) return SLA_ERR_NO_MEMORY;
    if (hipGetDevice(&h->device) != hipSuccess) {
        delete h;
        return SLA_ERR_DEVICE;
    }
    h->n = n;
    h->nnz = nnz;
    h->batch = batch;
    h->dtype = dtype;
    h->itype = row_ptr_type;
    h->rp = d_row_ptr;
    h->col = d_col;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    sla_status st = dispatch(h, [&](auto t, auto it) {
        using T = std::remove_pointer_t<decltype(t)>;
        using IT = std::remove_pointer_t<decltype(it)>;
        return create_typed<T, IT>(h, flags, s);
    });
    if (st != SLA_OK) {
        if (st == SLA_ERR_DEVICE && g_last_error == hipErrorOutOfMemory) st = SLA_ERR_NO_MEMORY;
        (void)hipStreamSynchronize(s);
        release(h);
        return st;
    }
    *out = h;
    return SLA_OK;
}

sla_status sla_destroy(sla_handle h) {
    if (!h) return SLA_ERR_ARG;
    DeviceGuard g(h->device);
    (void)hipDeviceSynchronize();
    release(h);
    return SLA_OK;
}

sla_status sla_matvec(sla_handle h, const void *d_values, const void *d_x, void *d_y,
                      int32_t transpose, void *stream) {
    if (!h || !d_values || !d_x || !d_y || d_x == d_y) return SLA_ERR_ARG;
    if (transpose && !h->has_t) return SLA_ERR_ARG;
    DeviceGuard g(h->device);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return dispatch(h, [&](auto t, auto it) -> sla_status {
        using T = std::remove_pointer_t<decltype(t)>;
        using IT = std::remove_pointer_t<decltype(it)>;
        for (int64_t s0 = 0; s0 < h->batch; s0 += 65535) {
            const int nb = (int)((h->batch - s0) < 65535 ? (h->batch - s0) : 65535);
            const T *v = reinterpret_cast<const T *>(d_values) + s0 * h->nnz;
            const T *x = reinterpret_cast<const T *>(d_x) + s0 * h->n;
            T *y = reinterpret_cast<T *>(d_y) + s0 * h->n;
            if (transpose)
                HIP_TRY((product_backward<T, IT>(h, v, nullptr, x, y, nullptr, nb, s)));
            else
                HIP_TRY((launch_spmv<T, IT>(h->slots, reinterpret_cast<const IT *>(h->rp), h->ca,
                                            v, h->nnz, x, y, h->n, h->n, nb, s, &h->plan)));
        }
        return SLA_OK;
    });
}

sla_status sla_matvec_adjoint(sla_handle h, const void *d_values, const void *d_x,
                              const void *d_grad_y, void *d_grad_x, void *d_grad_values,
                              void *stream) {
    if (!h || !d_values || !d_grad_y || (!d_grad_x && !d_grad_values)) return SLA_ERR_ARG;
    if (d_grad_x && (!h->has_t || d_grad_x == d_grad_y)) return SLA_ERR_ARG;
    if (d_grad_values && !d_x) return SLA_ERR_ARG;
    DeviceGuard g(h->device);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return dispatch(h, [&](auto t, auto it) -> sla_status {
        using T = std::remove_pointer_t<decltype(t)>;
        using IT = std::remove_pointer_t<decltype(it)>;
        for (int64_t s0 = 0; s0 < h->batch; s0 += 65535) {
            const int nb = (int)((h->batch - s0) < 65535 ? (h->batch - s0) : 65535);
            const T *v = reinterpret_cast<const T *>(d_values) + s0 * h->nnz;
            const T *gy = reinterpret_cast<const T *>(d_grad_y) + s0 * h->n;
            T *gx = d_grad_x ? reinterpret_cast<T *>(d_grad_x) + s0 * h->n : nullptr;
            T *gv = d_grad_values ? reinterpret_cast<T *>(d_grad_values) + s0 * h->nnz : nullptr;
            const T *x = d_x ? reinterpret_cast<const T *>(d_x) + s0 * h->n : nullptr;
            HIP_TRY((product_backward<T, IT>(h, v, x, gy, gx, gv, nb, s)));
        }
        return SLA_OK;
    });
}

sla_status sla_solve(sla_handle h, const void *d_values, const void *d_b, void *d_x,
                     const sla_solve_opts *opts, sla_solve_info *info, void *stream) {
    if (!h || !d_values || !d_b || !d_x || d_b == d_x) return SLA_ERR_ARG;
    const sla_solve_opts o = opts ? *opts : default_opts();
    if (check_opts(o) != SLA_OK) return SLA_ERR_ARG;
    DeviceGuard g(h->device);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return dispatch(h, [&](auto t, auto it) -> sla_status {
        using T = std::remove_pointer_t<decltype(t)>;
        using IT = std::remove_pointer_t<decltype(it)>;
        Operator op{h->rp, h->ca, h->slots, h->ia, h->it_slots, &h->plan};
        return solve_all<T, IT>(h, op, reinterpret_cast<const T *>(d_values),
                                reinterpret_cast<const T *>(d_b), reinterpret_cast<T *>(d_x), o,
                                info, s);
    });
}

sla_status sla_solve_adjoint(sla_handle h, const void *d_values, const void *d_x,
                             const void *d_grad_x, void *d_grad_values, void *d_grad_b,
                             const sla_solve_opts *opts, sla_solve_info *info, void *stream) {
    if (!h || !d_values || !d_x || !d_grad_x || !d_grad_values || !d_grad_b) return SLA_ERR_ARG;
    if (d_grad_b == d_grad_x || d_grad_b == d_x || d_grad_b == d_values) return SLA_ERR_ARG;
    const sla_solve_opts o = opts ? *opts : default_opts();
    if (check_opts(o) != SLA_OK) return SLA_ERR_ARG;
    if (o.method == SLA_BICGSTAB && !h->has_t) return SLA_ERR_ARG;
    DeviceGuard g(h->device);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return dispatch(h, [&](auto t, auto it) -> sla_status {
        using T = std::remove_pointer_t<decltype(t)>;
        using IT = std::remove_pointer_t<decltype(it)>;
        return adjoint_all<T, IT>(h, reinterpret_cast<const T *>(d_values),
                                  reinterpret_cast<const T *>(d_x),
                                  reinterpret_cast<const T *>(d_grad_x),
                                  reinterpret_cast<T *>(d_grad_values), reinterpret_cast<T *>(d_grad_b),
                                  o, info, s);
    });
}

sla_status sla_eigsh(sla_handle h, const void *d_values, double *h_evals, void *d_evecs,
                     const sla_eig_opts *opts, int32_t *h_restarts, void *stream) {
    if (!h || !d_values || !h_evals || !d_evecs || !opts) return SLA_ERR_ARG;
    const sla_eig_opts o = *opts;
    if (o.k < 1 || o.k > 8 || o.k > h->n || o.ncv < 0 || o.ncv > 512 || o.max_restarts < 0 ||
        !(o.tol > 0.0))
        return SLA_ERR_ARG;
    int m = o.ncv ? o.ncv : (4 * o.k > 40 ? 4 * o.k : 40);
    if (m > h->n) m = (int)h->n;
    if (m < o.k) return SLA_ERR_ARG;
    DeviceGuard g(h->device);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return dispatch(h, [&](auto t, auto it) -> sla_status {
        using T = std::remove_pointer_t<decltype(t)>;
        using IT = std::remove_pointer_t<decltype(it)>;
        EigWork wk;
        HIP_TRY(eig_buffers<T>(h, m, o.k, &wk));
        sla_status worst = SLA_OK;
        for (int64_t sys = 0; sys < h->batch; ++sys) {
            sla_status st = eigsh_one<T, IT>(
                h, reinterpret_cast<const T *>(d_values) + sys * h->nnz, o, m,
                h_evals + sys * o.k, reinterpret_cast<T *>(d_evecs) + sys * o.k * h->n,
                h_restarts ? h_restarts + sys : nullptr, wk, s);
            if (st < 0) return st;
            if (st > worst) worst = st;
        }
        return worst;
    });
}

sla_status sla_eigsh_adjoint(sla_handle h, const void *d_evecs, const void *d_grad_evals,
                             int32_t k, void *d_grad_values, void *stream) {
    if (!h || !d_evecs || !d_grad_evals || !d_grad_values || k < 1 || k > 8) return SLA_ERR_ARG;
    DeviceGuard g(h->device);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return dispatch(h, [&](auto t, auto it) -> sla_status {
        using T = std::remove_pointer_t<decltype(t)>;
        using IT = std::remove_pointer_t<decltype(it)>;
        for (int64_t sys = 0; sys < h->batch; ++sys)
            HIP_TRY((launch_eig_outer<T, IT>(
                reinterpret_cast<const IT *>(h->rp), h->col,
                reinterpret_cast<const T *>(d_evecs) + sys * k * h->n, k,
                reinterpret_cast<const T *>(d_grad_evals) + sys * k,
                reinterpret_cast<T *>(d_grad_values) + sys * h->nnz, h->n, s)));
        return SLA_OK;
    });
}

int32_t sla_column_mode(sla_handle h, int32_t transpose) {
    if (!h || (transpose && !h->has_t)) return -1;
    return transpose ? h->ca_t.mode : h->ca.mode;
}

int32_t sla_iteration_form(sla_handle h, int32_t transpose) {
    if (!h || (transpose && !h->has_t)) return -1;
    return transpose ? h->ia_t.mode : h->ia.mode;
}

sla_status sla_export_pattern(sla_handle h, void *d_diagpos, void *d_row_ptr_t, void *d_col_t,
                              void *d_perm, void *stream) {
    if (!h) return SLA_ERR_ARG;
    if ((d_row_ptr_t || d_col_t || d_perm) && !h->has_t) return SLA_ERR_ARG;
    DeviceGuard g(h->device);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const size_t isz = h->itype == SLA_I64 ? 8 : 4;
    if (d_diagpos)
        HIP_TRY(hipMemcpyAsync(d_diagpos, h->diagpos, isz * h->n, hipMemcpyDeviceToDevice, s));
    if (d_row_ptr_t)
        HIP_TRY(hipMemcpyAsync(d_row_ptr_t, h->rp_t, isz * (h->n + 1), hipMemcpyDeviceToDevice, s));
    if (d_col_t)
        HIP_TRY(hipMemcpyAsync(d_col_t, h->col_t, 4 * h->nnz, hipMemcpyDeviceToDevice, s));
    if (d_perm) HIP_TRY(hipMemcpyAsync(d_perm, h->perm, 4 * h->nnz, hipMemcpyDeviceToDevice, s));
    return SLA_OK;
}

int64_t sla_workspace_bytes(sla_handle h) { return h ? h->ws_bytes : -1; }

const char *sla_status_string(int32_t status) {
    switch (status) {
        case SLA_OK: return "ok";
        case SLA_NOT_CONVERGED: return "not converged (maxit reached)";
        case SLA_BREAKDOWN: return "breakdown (a Krylov denominator vanished)";
        case SLA_ERR_ARG: return "invalid argument";
        case SLA_ERR_PATTERN: return "invalid CSR pattern";
        case SLA_ERR_ZERO_DIAG: return "zero diagonal entry with Jacobi preconditioning";
        case SLA_ERR_NO_MEMORY: return "device out of memory";
        case SLA_ERR_DEVICE: return "HIP runtime error";
        case SLA_ERR_TOO_LARGE:
            return "beyond the no-alloc solve's fixed scratch (n <= 4096, batch <= 65535)";
        default: return "unknown status";
    }
}

const char *sla_last_error(void) { return hipGetErrorString(g_last_error); }

}  // extern "C"
