/*
 * sla.h -- C ABI of the MI355X (gfx950) differentiable sparse linear solve.
 *
 * The operation (torch-sla explainer pages, gist.science, "Technical summary"):
 *   forward   x = A^-1 b for a CSR matrix A, by Jacobi-preconditioned CG (SPD A)
 *             or BiCGStab (nonsymmetric A) -- Methodology section 1 names the
 *             iterative solvers, the Significance section the Jacobi
 *             preconditioner of the native backend;
 *   backward  one adjoint solve A^T lambda = dL/dx, then dL/db = lambda and
 *             dL/dA_ij = -lambda_i x_j on the stored pattern only --
 *             Methodology section 2, linear systems; memory stays O(n + nnz)
 *             whatever the iteration count (same section, complexity bullet);
 *   batching  one pattern shared by a batch of value arrays (Methodology
 *             section 1, "SparseTensor: single matrix / shared pattern").
 *
 * Conventions shared by every call
 *   - All d_* pointers are device pointers on the current HIP device.  Arrays
 *     are dense and contiguous, system-major: values [batch][nnz] in CSR order,
 *     vectors [batch][n].  The float type (SLA_F32 / SLA_F64) is fixed at
 *     sla_create and applies to every value and vector argument.
 *   - row_ptr is int32 or int64 (fixed at create); col is always int32.  The
 *     pattern must have row_ptr[0] = 0, non-decreasing row_ptr,
 *     row_ptr[n] = nnz, columns in [0, n) strictly ascending in each row, and
 *     every diagonal entry stored.
 *   - The pattern arrays are BORROWED: the caller keeps d_row_ptr and d_col
 *     alive and unchanged until sla_destroy.  The handle owns everything it
 *     derives (diagonal index, transpose map, solver workspace); nothing is
 *     allocated after sla_create and nothing grows with the iteration count.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     on it.  sla_solve and sla_solve_adjoint return after the solve has
 *     finished (they poll a device-resident convergence flag and read the
 *     per-system results); sla_matvec returns without synchronizing.
 *   - One handle serves one stream at a time; calls on a handle must not
 *     overlap.  Different handles are independent.
 *   - Errors are returned, never thrown or aborted across the ABI.  Argument
 *     and pattern errors are detected before any solver kernel is launched.
 */
#ifndef SLA_H
#define SLA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sla_ctx *sla_handle;

enum { SLA_F32 = 0, SLA_F64 = 1 };                 /* value / vector type   */
enum { SLA_I32 = 0, SLA_I64 = 1 };                 /* row_ptr index type    */
enum { SLA_CG = 0, SLA_BICGSTAB = 1 };             /* Krylov method         */
enum { SLA_PRECOND_NONE = 0, SLA_PRECOND_JACOBI = 1 };
/* sla_create flags */
enum { SLA_CREATE_TRANSPOSE = 1, SLA_CREATE_WIDE_COLUMNS = 2, SLA_CREATE_CSR_VALUES = 4 };

typedef enum {
    SLA_OK = 0,
    SLA_NOT_CONVERGED = 1,  /* maxit reached: x holds the maxit-th iterate  */
    SLA_BREAKDOWN = 2,      /* CG: p.Ap <= 0; BiCGStab: rhat.r, rhat.v, t.t
                               or t.s vanished; x holds the last iterate    */
    SLA_ERR_ARG = -1,       /* bad argument (NULL, size, type, option)      */
    SLA_ERR_PATTERN = -2,   /* invalid CSR pattern (see conventions)        */
    SLA_ERR_ZERO_DIAG = -3, /* Jacobi requested and some A_ii == 0          */
    SLA_ERR_NO_MEMORY = -4, /* device allocation failed at sla_create       */
    SLA_ERR_DEVICE = -5,    /* a HIP runtime call failed                    */
    SLA_ERR_TOO_LARGE = -6  /* sla_solve_noalloc: n or batch beyond the
                               fixed scratch (n <= 4096, batch <= 65535)    */
} sla_status;

/* Solver options.  Pass NULL for the defaults in brackets. */
typedef struct {
    double tol;          /* stop when ||r_k||_2 <= tol * ||rhs||_2 [1e-10]     */
    int32_t maxit;       /* iteration cap (>= 0) [1000]                        */
    int32_t method;      /* SLA_CG or SLA_BICGSTAB [SLA_CG]                    */
    int32_t precond;     /* SLA_PRECOND_JACOBI or _NONE [JACOBI]; BiCGStab
                            supports NONE only                                  */
    int32_t use_x0;      /* 1: d_x holds the initial guess; 0: start at 0 [0]  */
    int32_t graph_chunk; /* iterations per captured HIP graph replay for
                            large systems, > 0 = replays of that length,
                            < 0 = kernels launched directly in chunks of
                            that length (the host polls once per chunk),
                            0 = default: chunks of 16 (32 or 64 when the
                            handle's previous grid solve took at least 460
                            or 1800 iterations), launched directly when a
                            launch of the fused iterations advances at
                            least 32768 rows (CG) or 65536 (BiCGStab) in
                            all, else as graph replays                    */
    int32_t profile;     /* 1: no graph; time every launch of the fused SpMV
                            kernel with HIP events on `stream` (slower)       */
} sla_solve_opts;

/*
 * Per-call results.  The array members are HOST arrays of `batch` entries
 * (each may be NULL); the scalar members are filled in always.
 */
typedef struct {
    int32_t *iters;   /* iterations done per system (BiCGStab: started
                         iterations, a half-step exit counts as one)           */
    int32_t *spmv;    /* products with A (or A^T) per system                   */
    double *relres;   /* recurrence residual ||r||/||rhs|| per system          */
    int32_t *status;  /* sla_status per system                                  */
    double kernel_ms;        /* profile mode: summed duration of the fused
                                SpMV kernel launches (ms), else 0              */
    int64_t kernel_launches; /* profile mode: number of those launches         */
    int32_t form;     /* what the iterations read: the sla_iteration_form
                         codes 0-3, or 4 = diagonal-major with the entries
                         below the main diagonal read from their mirrors
                         above it (CG, mirrored offsets, values found
                         symmetric bit for bit in every system); -1 when
                         every system ran on the one-workgroup solver      */
} sla_solve_info;

/*
 * sla_create -- validate a CSR pattern and build its derived structures.
 *   n, nnz      matrix order and stored entries (n >= 1, nnz >= n; n < 2^31;
 *               nnz < 2^31 with SLA_I32 row_ptr)
 *   batch       number of value arrays / systems served by one call (>= 1)
 *   dtype       SLA_F32 or SLA_F64;  row_ptr_type  SLA_I32 or SLA_I64
 *   d_row_ptr   [n+1] device array of row_ptr_type (borrowed)
 *   d_col       [nnz] device int32 column indices (borrowed)
 *   flags       SLA_CREATE_TRANSPOSE: build the map of A^T (needed by
 *               sla_matvec with transpose = 1, by grad_x of
 *               sla_matvec_adjoint and by the BiCGStab adjoint): A^T's row
 *               pointers and rows, A's position of each A^T entry and A^T's
 *               position of each A entry (12 bytes per entry), and one
 *               system's buffer of nnz values; for patterns whose products
 *               read per-entry columns (no diagonal masks), 6 more bytes per
 *               entry: where the two-pass A^T products store each entry's
 *               term; requires nnz < 2^31.
 *               SLA_CREATE_WIDE_COLUMNS: read the caller's int32 columns in
 *               every product.  Without it the handle also keeps a compact
 *               copy (each column as an int16 offset from the first row of
 *               its 256-row tile, 2 bytes per entry) when every entry fits,
 *               and, for patterns on at most 16 diagonals with rows of at
 *               most 8 entries, one 16-bit diagonal mask per row; the
 *               products read the most compact form (sla_column_mode);
 *               results are identical.
 *               SLA_CREATE_CSR_VALUES: the solver iterations read the
 *               caller's CSR values.  Without it (and without
 *               SLA_CREATE_WIDE_COLUMNS), when the pattern's entries lie on
 *               3, 5 or 7 diagonals (nearest-neighbour stencils in 1, 2 and
 *               3 dimensions) and nd * n <= 1.25 nnz, the handle keeps a
 *               buffer of nd * n values per system of a launch group (see
 *               the workspace note below) and each grid-path solve first
 *               copies the systems' values into it
 *               diagonal-major, zero where a row lacks a diagonal; the
 *               iterations then read no row pointers or columns
 *               (sla_iteration_form).  CG on a system whose values are
 *               symmetric bit for bit (checked by the copy; the diagonals'
 *               offsets must pair up around the main one) reads only the
 *               main and upper diagonals, the lower entries through their
 *               mirrors (sla_solve_info.form = 4).  Results are identical as
 *               long as the iterates stay finite on systems of at most
 *               196 608 rows (768 tiles of 256); on larger ones the
 *               diagonal-major iterations run fewer workgroups (and, in
 *               fp64, two rows per lane), so their dot products add the
 *               same terms in another order and results agree to rounding.
 *               Other bits: SLA_ERR_ARG.
 * Workspace: CG and BiCGStab on a batch of systems with n > 4096 advance a
 * group of min(batch, 65535, 2^21 / n) systems (at least 1) per grid
 * launch, so the solver vectors (11 per system) and the diagonal-major
 * buffer are sized for that group; single systems, profile-mode solves and
 * the BiCGStab adjoint (which puts one system's values in A^T's order at a
 * time) use the first system's share.
 * Long rows: when some 256-row tile of A (or of A^T) holds more than 2048
 * entries or a row longer than 8, the handle keeps a row plan for it (short
 * row blocks and chunks of long rows, 32 bytes each, a flag per tile and one
 * partial sum per chunk of a split row and system, for up to 65535 systems);
 * the products, the gradient and CG (then three launches per iteration)
 * use it.  Building it reads the row pointers to the host once.
 * Checks the pattern on the device (synchronizes `stream`).  Returns
 * SLA_ERR_PATTERN for an invalid pattern and writes *out = NULL on failure.
 */
sla_status sla_create(sla_handle *out, int64_t n, int64_t nnz, int64_t batch,
                      int32_t dtype, int32_t row_ptr_type, const void *d_row_ptr,
                      const int32_t *d_col, int32_t flags, void *stream);

/* Release everything the handle owns (synchronizes the device). */
sla_status sla_destroy(sla_handle h);

/*
 * sla_matvec -- y[s] = A_s x[s] (transpose = 0) or A_s^T x[s] (transpose = 1)
 * for every system s of the batch.  d_values [batch][nnz], d_x and d_y
 * [batch][n]; d_y must not alias d_x.  Asynchronous on `stream`.
 * A^T x sums each row of A^T in ascending row order of A, every term
 * A_ij x_i rounded before it is added (bitwise the same through every
 * storage form and launch shape).  Without diagonal masks, a single system
 * (or any batch on a pattern of at least 2^20 entries) goes in two passes,
 * one system at a time: the terms are written to A^T's order in the
 * handle's buffer, then A^T's rows are summed; the product alone does so
 * while nnz * (2 * value size + 4) <= 192 MB, and beyond that reads A^T's
 * values through the transpose map (same bits).
 */
sla_status sla_matvec(sla_handle h, const void *d_values, const void *d_x,
                      void *d_y, int32_t transpose, void *stream);

/*
 * sla_matvec_adjoint -- backward pass of the differentiable product
 * y[s] = A_s x[s] (the autograd-aware .matvec of the unified API, torch-sla
 * explainer, Methodology section 1) for an upstream gradient
 * d_grad_y[s] = dL/dy:
 *   d_grad_x [batch][n]        = A_s^T grad_y[s]  (needs SLA_CREATE_TRANSPOSE;
 *                                 must not alias d_grad_y; bitwise the
 *                                 sla_matvec transpose = 1 result)
 *   d_grad_values [batch][nnz] = grad_y[s][row(k)] * x[s][col(k)] for every
 *                                 stored entry k (needs d_x)
 * Either output may be NULL (not both).  d_values, d_x, d_grad_y are inputs
 * of the layouts above.  SLA_ERR_ARG for a missing input, a missing transpose
 * map or aliasing.  Asynchronous on `stream`.
 */
sla_status sla_matvec_adjoint(sla_handle h, const void *d_values, const void *d_x,
                              const void *d_grad_y, void *d_grad_x,
                              void *d_grad_values, void *stream);

/*
 * sla_solve -- forward solve A_s x[s] = b[s] for every system.
 *   d_values [batch][nnz]; d_b [batch][n]; d_x [batch][n] output (input
 *   initial guess when opts->use_x0).  Per-system stopping: a converged system
 *   is frozen while the others continue.  Returns the most severe per-system
 *   status (errors < 0 first, then BREAKDOWN, then NOT_CONVERGED).
 */
sla_status sla_solve(sla_handle h, const void *d_values, const void *d_b,
                     void *d_x, const sla_solve_opts *opts,
                     sla_solve_info *info, void *stream);

/*
 * sla_solve_adjoint -- backward pass of x = A^-1 b for dL/dx = d_grad_x.
 *   Solves A_s^T lambda = grad_x[s] from lambda = 0 with the same method
 *   (CG uses A itself, which it presumes symmetric; BiCGStab uses the
 *   transpose map, so the handle needs build_transpose = 1), tol relative to
 *   ||grad_x[s]||.  Writes d_grad_b [batch][n] = lambda and
 *   d_grad_values [batch][nnz] = -lambda[row(k)] * x[col(k)] for every stored
 *   entry k (one gradient per stored entry, no symmetrisation).
 *   d_x is the forward solution.  d_grad_b must not alias any input.
 */
sla_status sla_solve_adjoint(sla_handle h, const void *d_values,
                             const void *d_x, const void *d_grad_x,
                             void *d_grad_values, void *d_grad_b,
                             const sla_solve_opts *opts, sla_solve_info *info,
                             void *stream);

/*
 * sla_solve_noalloc -- sla_solve for callers that cannot allocate device
 * memory (serving loops and harnesses that forbid allocation after start-up):
 * no handle, no hipMalloc, hipFree or allocating library call.
 *   The pattern (d_row_ptr [n+1] of row_ptr_type, d_col [nnz] int32) and
 *   d_values [batch][nnz], d_b [batch][n], d_x [batch][n] (output; input
 *   initial guess when opts->use_x0) are as for sla_create and sla_solve;
 *   the pattern is validated on every call (SLA_ERR_PATTERN).
 *   Only CG (opts->method = SLA_CG, Jacobi or no preconditioner, profile 0)
 *   on the one-workgroup solver: n <= 4096 and batch <= 65535, else
 *   SLA_ERR_TOO_LARGE; results (x and info) are those of sla_solve on a
 *   handle of the same pattern, bit for bit.
 *   Its state lives in a device array of 8 683 776 bytes that each
 *   device holds from the library's load until the process ends; every call
 *   on a device shares it, so calls that overlap on one device (two streams
 *   or two threads) race and must be serialized by the caller.  Synchronizes
 *   `stream` (three times: after the row-pointer check, after the column
 *   check, at the end).
 */
sla_status sla_solve_noalloc(int64_t n, int64_t nnz, int64_t batch, int32_t dtype,
                             int32_t row_ptr_type, const void *d_row_ptr,
                             const int32_t *d_col, const void *d_values, const void *d_b,
                             void *d_x, const sla_solve_opts *opts, sla_solve_info *info,
                             void *stream);

/*
 * Options of sla_eigsh.
 *   k             eigenpairs wanted, 1..8
 *   largest       0: the k smallest (algebraic) eigenvalues, 1: the k largest
 *   ncv           Lanczos basis per cycle, k..512 (0: max(4k, 40)), at most n
 *   max_restarts  explicit restarts after the first cycle (>= 0)
 *   tol           a Ritz pair (theta, x) is accepted when
 *                 ||A x - theta x|| <= tol * max |theta| over the wanted ones
 */
typedef struct {
    int32_t k;
    int32_t largest;
    int32_t ncv;
    int32_t max_restarts;
    double tol;
} sla_eig_opts;

/*
 * sla_eigsh -- extreme eigenpairs of each system's symmetric A_s (the
 * .eigsh of the unified API, torch-sla explainer, Methodology section 1), by
 * Lanczos with full reorthogonalisation and explicit restarts.  Writes
 * h_evals [batch][k] (host, ascending for the smallest, descending for the
 * largest) and d_evecs [batch][k][n] (device, unit 2-norm, sign arbitrary);
 * h_restarts [batch] (host, may be NULL) gets the restarts used.  The
 * symmetry of A is the caller's promise.  The handle keeps the basis
 * ((ncv + 1) * n values, ncv at most 512) from the first call until
 * sla_destroy and reallocates it only for a call with a larger basis or k
 * than any before (the one exception to "nothing is allocated after
 * sla_create"); synchronizes `stream`.  Returns SLA_NOT_CONVERGED when some
 * system did not meet tol.
 */
sla_status sla_eigsh(sla_handle h, const void *d_values, double *h_evals, void *d_evecs,
                     const sla_eig_opts *opts, int32_t *h_restarts, void *stream);

/*
 * sla_eigsh_adjoint -- gradient of sum_q g[s][q] lambda_q(A_s) with respect
 * to the stored values, by the Hellmann-Feynman theorem for simple
 * eigenvalues (torch-sla explainer, Methodology section 2, eigenvalue
 * problems: dlambda/dA_ij = v_i v_j on the pattern):
 *   d_grad_values[s][k'] = sum_q g[s][q] v_q[row(k')] v_q[col(k')].
 * d_evecs [batch][k][n] as written by sla_eigsh, d_grad_evals [batch][k]
 * (device, value dtype).  Asynchronous on `stream`.
 */
sla_status sla_eigsh_adjoint(sla_handle h, const void *d_evecs, const void *d_grad_evals,
                             int32_t k, void *d_grad_values, void *stream);

/*
 * sla_column_mode -- how the products read the columns of A (transpose = 0)
 * or of A^T (transpose = 1): 0 the caller's int32 array, 1 the compact
 * int16 tile-relative copy, 2 per-row masks over at most 16 diagonals (a
 * pattern whose entries lie on at most 16 diagonals, rows of at most 8
 * entries: 2 bytes per row).  -1 for a NULL handle or a missing transpose.
 */
int32_t sla_column_mode(sla_handle h, int32_t transpose);

/*
 * sla_iteration_form -- the form the solver iterations of the grid path read
 * for A (transpose = 0) or for A^T (transpose = 1, BiCGStab adjoint): the
 * sla_column_mode codes 0-2, or 3 for diagonal-major values (see
 * SLA_CREATE_CSR_VALUES).  -1 for a NULL handle or a missing transpose.
 */
int32_t sla_iteration_form(sla_handle h, int32_t transpose);

/*
 * sla_export_pattern -- copy the derived pattern structures into caller
 * device buffers (any pointer may be NULL): d_diagpos [n] (row_ptr type),
 * and, if the transpose was built, d_row_ptr_t [n+1] (row_ptr type),
 * d_col_t [nnz] int32 (row of each A^T entry) and d_perm [nnz] int32 (A's
 * position of each A^T entry).  Asynchronous on `stream`.
 */
sla_status sla_export_pattern(sla_handle h, void *d_diagpos, void *d_row_ptr_t,
                              void *d_col_t, void *d_perm, void *stream);

/* Device bytes owned by the handle (constant after sla_create, but for the
 * eigensolver basis that sla_eigsh adds). */
int64_t sla_workspace_bytes(sla_handle h);

/* Static description of a status code. */
const char *sla_status_string(int32_t status);

/* Text of the last HIP runtime error seen by this thread (after SLA_ERR_DEVICE). */
const char *sla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SLA_H */
