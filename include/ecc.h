/*
 * ecc.h -- C ABI of libecc_mi355.so: Euler characteristic curves of dense 2D/3D
 * grids on AMD Instinct MI355X (gfx950).
 *
 * Method: page "Scalable GPU-Accelerated Euler Characteristic Curves:
 * Optimization and Differentiable Learning for PyTorch" (paper notes),
 * section "Method / Key designs":
 *   - full-sweep kernel: every voxel's local contribution lands in an
 *     H-bin histogram kept per workgroup, flushed once per bin to global
 *     memory, and the curve is the running sum of that histogram;
 *   - local Euler-coefficient computation: chi splits into per-voxel
 *     contributions that need only a voxel's neighbourhood;
 *   - differentiable ECC layer: the hard sublevel indicator of
 *     value <= tau is replaced by a sigmoid of lambda*(tau - value), with an
 *     analytic backward pass for the thresholds.
 *
 * The complex: the grid's voxels are the vertices of a cubical complex.  Voxel
 * p owns its vertex and the edges, squares and (3D) cube that reach from p
 * towards +x, +y (, +z) and lie inside the grid.  A cell's value is the max
 * of its corner values; its sign is (-1)^dim.
 *
 * Conventions shared by every entry point:
 *   - Grids are C-contiguous, x (last index) fastest: grid[ny][nx] or
 *     grid[nz][ny][nx].  Any base alignment is accepted; 16-byte-aligned
 *     bases with a row pitch that is a multiple of 16 bytes take the fast
 *     vector-load path.
 *   - All pointers except `shape` are DEVICE pointers owned by the caller.
 *     The library allocates nothing per call and keeps no per-call state.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work and return; outputs are valid once the stream reaches
 *     that point.  Calls that share one workspace must not overlap in time.
 *   - Workspace: `ws` must hold the bytes its size function gives
 *     (ecc_workspace_bytes, ecc_workspace_bytes_batched or
 *     ecc_height_workspace_bytes for the call).  Before its
 *     FIRST use it must be zero-filled by the caller (e.g. torch.zeros);
 *     every call leaves it zero-filled again when it completes, so it can be
 *     reused by the next call on the same stream without clearing.
 *   - Errors: every entry point returns ECC_OK or an ECC_E_* code.  Argument
 *     errors are detected on the host before anything is enqueued; a launch
 *     failure returns ECC_E_HIP.  ecc_last_error() returns a thread-local
 *     message for the last failing call.  Nothing is printed and no C++
 *     exception crosses the ABI.
 *   - Not checked (documented preconditions): no grid value is NaN (+-inf
 *     are ordered like any other value: a cell at +inf enters only at a
 *     threshold of +inf); buffers are large enough for the shape given.
 */
#ifndef ECC_MI355_H
#define ECC_MI355_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define ECC_OK 0
#define ECC_E_NULL 1      /* a required pointer is NULL                      */
#define ECC_E_SHAPE 2     /* ndim not 2/3, a dimension or batch < 1, tau_stride < 0, or too many voxels */
#define ECC_E_DTYPE 3     /* dtype is not ECC_U8 / ECC_F32                    */
#define ECC_E_NTHRESH 4   /* H < 1 or H > ECC_MAX_THRESHOLDS                  */
#define ECC_E_LAMBDA 5    /* lambda not finite or <= 0                        */
#define ECC_E_WORKSPACE 6 /* ws is NULL or ws_bytes is too small              */
#define ECC_E_HIP 7       /* the HIP runtime reported an error               */
#define ECC_E_NDIRS 8     /* D < 1 or D > ECC_MAX_DIRECTIONS                  */

/* grid element types */
#define ECC_U8 0
#define ECC_F32 1

/* operations, for ecc_workspace_bytes */
#define ECC_OP_HARD 0
#define ECC_OP_SOFT_FWD 1
#define ECC_OP_SOFT_BWD 2

#define ECC_MAX_THRESHOLDS 8192
#define ECC_MAX_VOXELS (((int64_t)1) << 40)
#define ECC_MAX_DIRECTIONS 4096
#define ECC_MAX_AXIS (((int64_t)1) << 24) /* per axis, for the directional heights */

/*
 * Hard ECC of a 2D grid (full-sweep kernel).
 *   grid    device, dtype elements, [ny][nx]
 *   tau     device float32[H]: the thresholds
 *   out     device int64[H]:   out[k] = sum over cells c of (-1)^dim(c) *
 *           [bin(c) <= k], where bin(c) = min{j : value(c) <= tau_j} with an
 *           exact IEEE float32 comparison (uint8 values are widened exactly).
 *           For non-decreasing tau, out[k] is the Euler characteristic of the
 *           sublevel complex {c : value(c) <= tau_k}; for any other order it
 *           is that of the running maximum of tau_0..tau_k.
 *   ws      device workspace, see the conventions above.
 * One kernel launch.  Result bit-exact (integer arithmetic throughout).
 */
int ecc_hard_2d(const void* grid, int dtype, int64_t ny, int64_t nx, const float* tau, int32_t H,
                int64_t* out, void* ws, size_t ws_bytes, void* stream);

/*
 * Hard ECC of a 3D grid [nz][ny][nx]; otherwise as ecc_hard_2d.
 * Speed (not results) depends on the thresholds for float32 grids: finite,
 * roughly evenly spaced thresholds (e.g. linspace(min, max, H)) bin through an
 * exact one-read table; thresholds that crowd together (e.g. data quantiles)
 * take a short per-bucket scan or a binary search, about 2x-6x slower.
 */
int ecc_hard_3d(const void* grid, int dtype, int64_t nz, int64_t ny, int64_t nx, const float* tau,
                int32_t H, int64_t* out, void* ws, size_t ws_bytes, void* stream);

/*
 * ecc_hard_3d without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation).  Same arguments, result and errors as ecc_hard_3d
 * (a 2D grid is nz = 1) minus `ws` / `ws_bytes`: the workspace is a static
 * device array inside the library, 529 KB (the tickets and accumulators of
 * any H <= ECC_MAX_THRESHOLDS), one copy per GPU, held until the process
 * ends.  The call allocates nothing; its first call on a device looks the
 * array up and clears it with a kernel on `stream`, and every call leaves it
 * zero.  All calls on one GPU share that array: calls that overlap on one GPU
 * (other streams, other threads) race and must be serialized by the caller.
 * A size the array cannot serve is rejected with ECC_E_WORKSPACE.
 */
int ecc_hard_3d_static(const void* grid, int dtype, int64_t nz, int64_t ny, int64_t nx, const float* tau,
                       int32_t H, int64_t* out, void* stream);

/*
 * Hard ECC of a batch of `batch` 2D grids of one shape, stored back to back:
 * grid[batch][ny][nx].  Grid b is binned against tau + b * tau_stride
 * (tau_stride = 0: one float32[H] threshold array for every grid; H: one row
 * of a float32[batch][H] array per grid) and its curve, defined as for
 * ecc_hard_2d, goes to out[b][0..H) (int64[batch][H]).
 *   ws  device workspace of ecc_workspace_bytes_batched(ECC_OP_HARD, batch, H)
 *       bytes, zero-filled before first use, left zero-filled by every call.
 * Batched execution is what the page lists as missing for training-scale use
 * (section "Limitations and outlook"): one small grid cannot fill the GPU, a
 * batch can.  Each grid gets its own workgroups, so the result equals that of
 * `batch` separate calls, bit for bit.  One kernel launch per 65535 grids.
 */
int ecc_hard_2d_batched(const void* grid, int dtype, int64_t batch, int64_t ny, int64_t nx,
                        const float* tau, int64_t tau_stride, int32_t H, int64_t* out, void* ws,
                        size_t ws_bytes, void* stream);

/* Batched hard ECC of 3D grids grid[batch][nz][ny][nx]; otherwise as ecc_hard_2d_batched. */
int ecc_hard_3d_batched(const void* grid, int dtype, int64_t batch, int64_t nz, int64_t ny, int64_t nx,
                        const float* tau, int64_t tau_stride, int32_t H, int64_t* out, void* ws,
                        size_t ws_bytes, void* stream);

/*
 * Soft ECC forward (differentiable ECC layer).
 *   grid    device float32, ndim in {2,3}, shape[ndim] (HOST array, slowest first)
 *   tau     device float32[H]; lambda > 0 and finite (inverse temperature)
 *   out     device float32[H]: out[k] = sum_c (-1)^dim(c) *
 *           sigmoid(lambda * (tau_k - value(c))), sigmoid(z) = 1/(1+exp(-z)).
 * Sigmoids are evaluated in float32 and summed in float64 per workgroup;
 * workgroup sums are combined in 64-bit fixed point (resolution 2^-s with
 * s = 61 - ceil(log2(8*voxels+8)), e.g. 2^-33 at 256^3), so the result
 * does not depend on scheduling.
 * Accuracy: |out[k] - exact| <= sum_c e_c sigmoid(x_c) + (W / 2) 2^-s
 * + |out[k]| 2^-24, where x_c = lambda (tau_k - value(c)), e_c = (6 + 1.5 |x_c|)
 * 2^-24 bounds the relative error of one float32 sigmoid (the exponent is
 * formed in float32 when the thresholds span more than 100 / (lambda log2 e)
 * either side of their middle, hence the |x_c| term), and W <= ceil(voxels /
 * 512) is the number of workgroups on the grid.  One kernel launch.
 */
int ecc_soft_fwd(const float* grid, int32_t ndim, const int64_t* shape, const float* tau, int32_t H,
                 float lambda, float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * Soft ECC backward with respect to the thresholds.
 *   grad_out  device float32[H]: dL/dout
 *   grad_tau  device float32[H]: OVERWRITTEN with dL/dtau_k =
 *             grad_out[k] * lambda * sum_c (-1)^dim(c) s(x)(1 - s(x)),
 *             x = lambda * (tau_k - value(c)), s = sigmoid.
 * (out[k] depends on tau_k only, so the Jacobian is diagonal.)  Same
 * arithmetic and determinism as ecc_soft_fwd; the sum is formed before the
 * scaling by lambda * grad_out[k], which therefore scales its error:
 * |grad_tau[k] - exact| <= lambda |grad_out[k]| (sum_c e_c s(x_c)(1 - s(x_c))
 * + (W / 2) 2^-s) + |grad_tau[k]| 2^-24 with e_c = (8 + 1.5 |x_c|) 2^-24 and
 * W, s as for ecc_soft_fwd.  Where the signed sum cancels and lambda
 * |grad_out[k]| is large, that can exceed a fixed absolute tolerance.  One
 * kernel launch.
 */
int ecc_soft_bwd_tau(const float* grid, int32_t ndim, const int64_t* shape, const float* tau,
                     int32_t H, float lambda, const float* grad_out, float* grad_tau, void* ws,
                     size_t ws_bytes, void* stream);

/*
 * Soft ECC backward with respect to the grid values.
 *   grad_out   device float32[H]: dL/dout
 *   grad_grid  device float32, the grid's shape: OVERWRITTEN with dL/dgrid.
 * A cell's value is the max of its corners, so its derivative goes to the
 * corner holding the max; among equal maxima, to the first in index order
 * (x fastest), i.e. one subgradient of the max.  Hence
 *   grad_grid[p] = -lambda * c(p) * sum_k grad_out[k] s(x)(1 - s(x)),
 *   x = lambda * (tau_k - grid[p]),  s = sigmoid,
 * with c(p) the sum of (-1)^dim(c) over the cells whose derivative goes to p
 * (cells met inside p's 3x3(x3) block; voxels with c(p) = 0 get 0).
 * Accuracy: every output is within max(9e-4, 9e-5 |exact|) of the exact
 * value.  The sum over thresholds runs in float32 terms with float64
 * accumulation and a per-voxel rounding-error bound; voxels whose bound could
 * exceed that (the terms cancel: large upstream gradients of both signs, or
 * large lambda |c(p)|) are recomputed in float64 from the formula above.
 * Every voxel is written exactly once, in a fixed order of operations, so
 * the result does not depend on scheduling.  Needs no workspace: it may run
 * concurrently with any other call that does not write its inputs.  The
 * values of grad_out are taken as finite.  One kernel launch.
 * (Section "Method / Key designs / differentiable ECC layer" gives the
 * relaxation; the gradient with respect to the grid follows from it.)
 */
int ecc_soft_bwd_grid(const float* grid, int32_t ndim, const int64_t* shape, const float* tau,
                      int32_t H, float lambda, const float* grad_out, float* grad_grid, void* stream);

/*
 * Batched soft ECC: `batch` grids of one shape `shape` (HOST array of ndim
 * entries, the shape of ONE grid), stored back to back.  Grid b uses
 * tau + b * tau_stride (0: shared thresholds) and, for the backward calls,
 * grad_out + b * H.  Outputs:
 *   ecc_soft_fwd_batched       out[b][k]        float32[batch][H]
 *   ecc_soft_bwd_tau_batched   grad_tau[b][k]   float32[batch][H], the
 *                              contribution of grid b (with shared thresholds
 *                              the gradient of tau is the sum over b)
 *   ecc_soft_bwd_grid_batched  grad_grid        float32[batch][shape...]
 * Each grid is computed with the arithmetic of the single-grid call; the
 * split of its cells among workgroups depends on the batch size, so the
 * curves agree with single calls to float64 rounding of the workgroup sums
 * (the grid gradient, one value per voxel, agrees bit for bit).  The workspace of the
 * first two is ecc_workspace_bytes_batched(ECC_OP_SOFT_*, batch, H) bytes,
 * with the zero-fill convention above; the grid gradient needs none.  One
 * kernel launch per 65535 grids.  Batches are how the differentiable layer
 * meets training-scale inputs (section "Limitations and outlook").
 */
int ecc_soft_fwd_batched(const float* grid, int32_t ndim, const int64_t* shape, int64_t batch,
                         const float* tau, int64_t tau_stride, int32_t H, float lambda, float* out, void* ws,
                         size_t ws_bytes, void* stream);
int ecc_soft_bwd_tau_batched(const float* grid, int32_t ndim, const int64_t* shape, int64_t batch,
                             const float* tau, int64_t tau_stride, int32_t H, float lambda,
                             const float* grad_out, float* grad_tau, void* ws, size_t ws_bytes,
                             void* stream);
/*
 * dL/dtau of thresholds shared by a whole batch: grid_tau[k] =
 *   sum over b of grad_out[b][k] * lambda * sum_{c in grid b} (-1)^dim(c) s(x)(1 - s(x)),
 * the gradient of the one threshold array every grid of the batch uses (the
 * batched differentiable layer with a learnable tau, section "Limitations and
 * outlook" of the page: batched execution).  Same arguments as
 * ecc_soft_bwd_tau_batched with tau_stride = 0, except
 *   grad_out  device float32[batch][H]
 *   grad_tau  device float32[H]: OVERWRITTEN with the sum over the batch.
 * The sum is formed on the device in a fixed order (each grid's float64
 * values, summed in grid order within groups of 64 grids, then over the
 * groups in order), so the result does not depend on scheduling.  Workspace:
 * ecc_workspace_bytes_batched(ECC_OP_SOFT_BWD, batch, H) bytes, zero-filled
 * convention as above.  One kernel launch per 65535 grids.
 */
int ecc_soft_bwd_tau_shared(const float* grid, int32_t ndim, const int64_t* shape, int64_t batch,
                            const float* tau, int32_t H, float lambda, const float* grad_out, float* grad_tau,
                            void* ws, size_t ws_bytes, void* stream);

int ecc_soft_bwd_grid_batched(const float* grid, int32_t ndim, const int64_t* shape, int64_t batch,
                              const float* tau, int64_t tau_stride, int32_t H, float lambda,
                              const float* grad_out, float* grad_grid, void* stream);

/*
 * Directional heights (single- and multi-direction curves).
 *   grid   device float32, ndim in {2,3}, shape[ndim] (HOST array); each axis <= 2^24
 *   dirs   device float32[D][ndim]: direction u_d, axis order slowest first
 *   alpha  device float32[D]: scale alpha_d
 *   out    device float32[D][shape...]: out[d][p] = grid[p] + alpha_d * <u_d, p>,
 *          p the integer voxel index, computed in float32 as
 *          h = (u_0 p_0 + u_1 p_1) [+ u_2 p_2], out = grid + alpha * h, each
 *          product and sum rounded in that order (no fused multiply-add).
 * The page's differentiable layer has a learnable direction u and scale alpha
 * for its single-direction version, and the multi-direction transform is its
 * complete form ("Method / Key designs / differentiable ECC layer",
 * "Limitations and outlook"); the page leaves the height on a grid open, and
 * this is the reading taken: intensity plus a linear ramp.  Voxels at +inf
 * never enter any sublevel set, so grid = 0 on a shape and +inf off it gives
 * the shape's directional filtration.  The curves of direction d are those of
 * out[d], e.g. from ecc_hard_2d/3d_batched or ecc_soft_fwd_batched with
 * batch = D.  One kernel launch; no workspace.
 */
int ecc_height(const float* grid, int32_t ndim, const int64_t* shape, const float* dirs, const float* alpha,
               int32_t D, float* out, void* stream);

/*
 * Backward of ecc_height.  grad_h: device float32[D][shape...] = dL/dout.
 *   grad_grid   device float32[shape...] or NULL: sum over d of grad_h[d]
 *               (float32, d increasing)
 *   grad_dirs   device float32[D][ndim] or NULL: alpha_d * M[d][i],
 *   grad_alpha  device float32[D] or NULL (both or neither): sum_i u_d,i M[d][i],
 *               with M[d][i] = sum_p grad_h[d][p] * p_i in float64, summed in a
 *               fixed order (the result does not depend on scheduling).
 *   ws          device workspace of ecc_height_workspace_bytes(ndim, D) bytes
 *               (needed with grad_dirs; zero-filled convention as above).
 * Up to two kernel launches (one per requested output kind).
 */
int ecc_height_bwd(const float* grad_h, int32_t ndim, const int64_t* shape, const float* dirs, const float* alpha,
                   int32_t D, float* grad_grid, float* grad_dirs, float* grad_alpha, void* ws, size_t ws_bytes,
                   void* stream);

/* Workspace bytes of ecc_height_bwd (0 for invalid arguments). */
size_t ecc_height_workspace_bytes(int32_t ndim, int32_t D);

/*
 * Bytes of workspace needed by an operation (ECC_OP_*) for a grid of `ndim`
 * dimensions `shape` (host array; may be NULL, the size does not depend on
 * it today) and H thresholds.  Returns 0 for invalid op/H.
 */
size_t ecc_workspace_bytes(int op, int32_t ndim, const int64_t* shape, int32_t H);

/*
 * Bytes of workspace for a batched operation (ECC_OP_*) over `batch` grids
 * with H thresholds: one slice per grid.  Returns 0 for invalid arguments.
 */
size_t ecc_workspace_bytes_batched(int op, int64_t batch, int32_t H);

/* Static text for a status code (never NULL). */
const char* ecc_status_string(int status);

/* Thread-local detail message of the last failing call on this thread ("" if none). */
const char* ecc_last_error(void);

/* Library version, e.g. "0.1.0". */
const char* ecc_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ECC_MI355_H */
