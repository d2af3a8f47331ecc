/*
 * spc.h -- C ABI of libspc: kernel maps and sparse 3-D convolution on voxel
 * coordinate sets, hand-written HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Coordinates are int32 rows (b, z, y, x), batch index first, as in spconv's
 *   SparseConvTensor (spconv USAGE.md, "Creating and Converting
 *   SparseConvTensor").  Rows may come in any order; no call reorders them.
 * - Kernel offsets are flattened z-slowest, k = (kz * KY + ky) * KX + kx, and
 *   output site o reads the input at o*stride - pad + k*dil per axis (torch
 *   conv3d cross-correlation; spconv USAGE.md, "Core Concepts": a sparse
 *   convolution equals the dense convolution of the densified tensor).  For a
 *   submanifold convolution this is the centred C-order offset list of the MLX
 *   sparse/conv.py page (_kernel_offsets) with stride 1 and pad ksize/2.
 * - Weights are [K, Cin, Cout] row-major (MLX sparse/conv.py page, SubMConv3d).
 * - feats / weight / out / dout / din share one dtype (spc_dtype); bias, dW and
 *   dbias are fp32.  Accumulation is fp32, and a 16-bit output is rounded once,
 *   round-to-nearest-even, from the fp32 accumulator with the bias added.
 * - Every pointer except n_out / out_shape / bytes (and the host arrays of
 *   spc_point_to_voxel) is a DEVICE pointer owned by the caller; the library
 *   allocates no device memory.  Its only state between calls is per host
 *   thread: an error string and, per device, created on first use, 64 bytes
 *   of pinned host memory with an event (for the strided kernel map's count).
 *   Device pointers must be 16-byte aligned.  Every launch is on `stream`
 *   (NULL = the default stream), in order.
 * - Errors: a call returns before any launch when its host-side checks fail,
 *   leaving outputs untouched; spc_last_error() then describes the failure.
 *   Only the strided spc_build_kmap (for the output count) and
 *   spc_point_to_voxel (for the voxel count) wait for the GPU, once each;
 *   every other call is asynchronous (spc_build_kmap_async is the kernel map
 *   that leaves its count in device memory instead of waiting).
 * - Sizes: row counts below 2^31; channel counts multiples of 16.
 */
#ifndef SPC_H
#define SPC_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum spc_status {
    SPC_OK = 0,
    SPC_ERR_ARG = 1,          /* a pointer, size or geometry argument is invalid   */
    SPC_ERR_UNSUPPORTED = 2,  /* valid, but outside what this library implements   */
    SPC_ERR_CAPACITY = 3,     /* out_cap too small; *n_out holds the count needed  */
    SPC_ERR_COORD = 4,        /* duplicate or out-of-range input coordinates       */
    SPC_ERR_WORKSPACE = 5,    /* ws_bytes below what the size query returned       */
    SPC_ERR_HIP = 6           /* a HIP runtime call failed                          */
} spc_status;

typedef enum spc_dtype { SPC_F32 = 0, SPC_F16 = 1, SPC_BF16 = 2 } spc_dtype;

/* Bits written to *coord_err by spc_build_kmap. */
#define SPC_COORD_OUT_OF_RANGE 1  /* b not in [0, batch) or z/y/x outside shape  */
#define SPC_COORD_DUPLICATE    2  /* two rows share (b, z, y, x)                  */

/* Input table of spc_build_kmap (spc_geom.table). */
#define SPC_TABLE_HASH 0  /* open-addressing hash over the packed keys, 2^ceil(log2 4N)
                             slots of 8 bytes (the default; any grid)               */
#define SPC_TABLE_GRID 1  /* occupancy bitmap (1 bit per cell, cleared per call) and an
                             int32 index grid (4 bytes per cell, never cleared) over
                             the whole input grid: batch*Z*Y*X*4.125 bytes of
                             workspace, for grids that are small next to N          */

/*
 * Convolution geometry.  subm != 0 selects a submanifold convolution (spconv
 * USAGE.md, "Submanifold Convolution": output sites are the input sites): each
 * ksize must be odd (the MLX page's SubMConv3d rejects even sizes), and stride,
 * pad and dil are ignored (1, ksize/2, 1).  subm == 0 selects a strided sparse
 * convolution whose output extent per axis is
 * floor((shape + 2*pad - dil*(ksize-1) - 1) / stride) + 1.
 * batch * Z * Y * X (and the output grid's volume) must stay below 2^32.
 * table selects the kernel map's input table (SPC_TABLE_*); both give the
 * same results bit for bit.
 */
typedef struct spc_geom {
    int32_t batch;      /* samples; coords[:,0] in [0, batch)           */
    int32_t shape[3];   /* input spatial extent (Z, Y, X)               */
    int32_t ksize[3];
    int32_t stride[3];
    int32_t pad[3];
    int32_t dil[3];
    int32_t subm;
    int32_t table;      /* SPC_TABLE_HASH (0) or SPC_TABLE_GRID          */
} spc_geom;

/* Host only.  Output spatial extent of a strided geometry (the input shape for
 * subm).  Extents <= 0 mean an empty output (spconv COMMON_PROBLEMS.md: the
 * [8,200,200] example whose only site is dropped along z). */
spc_status spc_out_shape(const spc_geom* g, int32_t out_shape[3]);

/* Host only.  Workspace bytes spc_build_kmap needs for n_in input rows. */
spc_status spc_kmap_workspace(const spc_geom* g, int64_t n_in, size_t* bytes);

/*
 * Kernel map ("indice pairs"; spconv's get_indice_pairs_implicit_gemm on the
 * context7 spconv page, INT8_GUIDE.md snippet).  Builds a GPU hash table over
 * the packed keys ((b*Z + z)*Y + y)*X + x of the input rows (the single-slot
 * hash.HashTable of the spconv page; g->table may select the index grid
 * instead) and probes it for every kernel offset.  Maps are row-major: entry
 * k of a row is that row's neighbour through offset k.
 *
 * subm != 0 (the MLX page's build_indice_map, computed on the GPU):
 *   nbr       [n_in, K] int32: nbr[i*K + k] = row j with coords[j] =
 *             coords[i] + d_k in the same sample, else -1.  *n_out = n_in.
 *   out_coords, out_cap, nbr_in, order_in: unused (may be NULL / 0).
 * subm == 0 (spconv USAGE.md, "Sparse Convolution"):
 *   out_coords [out_cap, 4] int32: the M output sites, sorted by (b, z, y, x).
 *   nbr       [M, K] int32 (a buffer of out_cap*K entries): input row read by
 *             output o through offset k, else -1.
 *   nbr_in    [n_in, K] int32 (NULL ok): output row fed by input i through
 *             offset k, else -1.
 *   *n_out    receives M.  The call waits once, for the count only: the maps,
 *             pair lists and orders are still being built in stream order
 *             when it returns.
 *   If out_coords is NULL the call only counts: *n_out = M, nothing else is
 *   written.  If M > out_cap it returns SPC_ERR_CAPACITY with *n_out = M.
 *   An empty output (M = 0) is valid.
 * Pair lists (both kinds; all three NULL or all three set): for each offset
 *   k, the pairs (nbr[o*K + k], o) with nbr[o*K + k] >= 0 in ascending o, as
 *   CSR: pair_ptr [K+1] int32 (offset k owns [pair_ptr[k], pair_ptr[k+1])),
 *   pair_in / pair_out [pair_cap] int32, pair_cap >= K * n_in.
 * Processing orders (NULL ok): order [rows of nbr] receives the rows of nbr
 *   sorted by their neighbour mask (bit k set iff entry k >= 0), ties by row
 *   index; order_in [n_in] (strided only) does the same for nbr_in.  The
 *   convolutions take these orders to gather rows with equal neighbour sets
 *   into the same tiles.  For K > 32 they are the identity.
 * coord_err (NULL ok): device int32 receiving SPC_COORD_* bits.  Rows flagged
 *   out of range are left out of the table; for a duplicate the map refers to
 *   one of the equal rows.  The strided call also returns SPC_ERR_COORD.
 * ws: device workspace of at least spc_kmap_workspace() bytes; its contents
 *   are scratch and need no initialisation.
 */
spc_status spc_build_kmap(const spc_geom* g, const int32_t* coords, int64_t n_in,
                          int32_t* out_coords, int64_t out_cap, int64_t* n_out,
                          int32_t* nbr, int32_t* nbr_in,
                          int32_t* pair_ptr, int32_t* pair_in, int32_t* pair_out, int64_t pair_cap,
                          int32_t* order, int32_t* order_in,
                          int32_t* coord_err, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * spc_build_kmap without any wait, for callers that capture a layer into a HIP
 * graph or keep the host free (the strided map of spconv USAGE.md, "Sparse
 * Convolution", whose output count only the GPU knows).  Arguments as
 * spc_build_kmap, except:
 *   n_out_dev  device int32 (16-byte aligned, required) that receives the
 *              output row count in stream order: M for a strided map, n_in
 *              for a submanifold one.  Nothing is copied to the host.
 *   out_coords must be set for a strided map (no count-only form).
 * Every launch reads M on the device; a map with M > out_cap holds no rows
 * (its kernels treat the count as 0), and *n_out_dev = M tells the caller
 * so.  Coordinate errors are reported only through coord_err (pass it).
 * The call itself allocates nothing and issues no memset or copy: kernels
 * only.
 */
spc_status spc_build_kmap_async(const spc_geom* g, const int32_t* coords, int64_t n_in,
                                int32_t* out_coords, int64_t out_cap, int32_t* n_out_dev,
                                int32_t* nbr, int32_t* nbr_in,
                                int32_t* pair_ptr, int32_t* pair_in, int32_t* pair_out, int64_t pair_cap,
                                int32_t* order, int32_t* order_in,
                                int32_t* coord_err, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Submanifold forward (the MLX page's module docstring formula):
 *   out[c] = bias + sum_k feats[nbr[c*K + k]] @ W[k]   over offsets with nbr >= 0.
 * feats [n, cin], weight [K, cin, cout], bias [cout] fp32 (NULL ok),
 * nbr [n, K] from spc_build_kmap, out [n, cout].  order (NULL ok) is the
 * processing order from spc_build_kmap; it changes only which rows share a
 * tile, never a result.  K == 1 is the per-voxel
 * linear layer out = feats @ W[0] + bias (MLX page, k=1 path; the Hygon
 * spconv-das README routes 1x1 convolutions to a GEMM); nbr may then be NULL.
 * One fused kernel: gathered rows feed MFMA tiles directly, the fp32
 * accumulator stays in registers per output row (no atomics, deterministic).
 */
spc_status spc_subm_conv_fwd(spc_dtype dtype, const void* feats, int64_t n, int32_t cin,
                             const void* weight, int32_t K, int32_t cout, const float* bias,
                             const int32_t* nbr, const int32_t* order, void* out, hipStream_t stream);

/*
 * Strided forward, the downsampling SparseConv3d (spconv USAGE.md,
 * "spconv.pytorch Core Concepts Definitions": a sparse convolution equals the
 * dense convolution of the densified tensor and computes only on valid data;
 * "spconv.pytorch Layer APIs Reference": SparseConv3d downsamples, dense
 * version nn.Conv3d):
 *   out[o] = bias + sum_k feats[nbr_out[o*K + k]] @ W[k]   over entries >= 0
 * for the n_out output rows of a strided spc_build_kmap.
 * feats [n_in, cin] (the map's input rows), weight [K, cin, cout], bias [cout]
 * fp32 (NULL ok), nbr_out [n_out, K] = that call's nbr, order (NULL ok) = its
 * order, out [n_out, cout] (overwritten; n_out may be 0).  Entries outside
 * [0, n_in) count as absent.  Errors: SPC_ERR_ARG for a NULL or misaligned
 * pointer or a negative size; SPC_ERR_UNSUPPORTED for channel counts that are
 * not multiples of 16 or a contraction beyond the kernels' limit (256 16-bit,
 * 128 fp32 channels).  One kernel on `stream`, asynchronous.
 */
spc_status spc_sparse_conv_fwd(spc_dtype dtype, const void* feats, int64_t n_in, int32_t cin,
                               const void* weight, int32_t K, int32_t cout, const float* bias,
                               const int32_t* nbr_out, const int32_t* order, int64_t n_out, void* out,
                               hipStream_t stream);

/*
 * Inverse (upsampling) forward, SparseInverseConv3d (spconv USAGE.md, the
 * layer table and "Using SparseInverseConv for Inverse Sparse Operations"):
 * the output rows are the INPUT sites of the strided layer whose kernel map
 * is reused, and
 *   out[i] = bias + sum_k feats[nbr_in[i*K + k]] @ W[k]   over entries >= 0.
 * feats [n_coarse, cin] lives on that layer's output sites; weight
 * [K, cin, cout] is the inverse layer's own; nbr_in [n_fine, K] and order_in
 * (NULL ok) come from the strided spc_build_kmap; out [n_fine, cout] is
 * overwritten.  Errors as spc_sparse_conv_fwd.
 * The backward needs no further entry point; with the same strided map:
 *   dinput  = spc_conv_bwd_input(dout [n_fine, cout], weight, map = that map's
 *             nbr [n_coarse, K], map_is_subm = 0, order = its order,
 *             n_in = n_coarse), i.e. din[o] = sum_k dout[nbr[o*K + k]] @ W[k]^T;
 *   dfilter = spc_conv_bwd_filter(feats = the coarse features, dout = the fine
 *             gradient, pair_in and pair_out of that map exchanged).
 */
spc_status spc_sparse_inverse_conv_fwd(spc_dtype dtype, const void* feats, int64_t n_coarse, int32_t cin,
                                       const void* weight, int32_t K, int32_t cout, const float* bias,
                                       const int32_t* nbr_in, const int32_t* order_in, int64_t n_fine,
                                       void* out, hipStream_t stream);

/*
 * Fused forward (the implicit-GEMM call on spconv TENSORRT_INT8_GUIDE.md, "Call
 * Spconv Implicit GEMM with Calculated Scales and Bias": a bias, an added
 * output and a ReLU activation fused into the convolution for a
 * conv-add-relu layer).  Any of the forwards above, with
 *   out[r] = act(bias + residual[r] + sum_k feats[map[r*K + k]] @ W[k])
 * all in fp32 with one rounding to the storage dtype; act is ReLU when
 * relu != 0 (NaN passes through), else the identity.
 * map [n_rows, K] is the submanifold nbr (n_src == n_rows), the strided nbr
 * (n_src = input rows) or the strided nbr_in for the inverse layer (n_src =
 * coarse rows); NULL with K == 1 is the identity (n_src == n_rows).  order as
 * for that map (NULL ok).  residual [n_rows, cout] in the features' dtype,
 * NULL for none; it may be the same buffer as out (in-place add).  Other
 * arguments and errors as spc_subm_conv_fwd.
 */
spc_status spc_conv_fwd_fused(spc_dtype dtype, const void* feats, int64_t n_src, int32_t cin,
                              const void* weight, int32_t K, int32_t cout, const float* bias,
                              const int32_t* map, const int32_t* order, int64_t n_rows,
                              const void* residual, int32_t relu, void* out, hipStream_t stream);

/*
 * Weight transpose for the forwards below: weight_t[k][n][c] = weight[k][c][n],
 * weight [K, cin, cout] -> weight_t [K, cout, cin], same dtype, device
 * memory owned by the caller; the two buffers must not overlap.  One kernel
 * on `stream`.  (The per-offset weight matrices of the MLX sparse/conv.py
 * page's formula, stored contraction-contiguous.)
 */
spc_status spc_transpose_weight(spc_dtype dtype, const void* weight, int32_t K, int32_t cin, int32_t cout,
                                void* weight_t, hipStream_t stream);

/*
 * spc_conv_fwd_fused with the weights given transposed, weight_t [K, cout,
 * cin] from spc_transpose_weight: the same result bit for bit.  The kernel
 * then stages each offset's weights as plain contraction-contiguous copies
 * instead of transposing them per tile, which pays for fp32 and for
 * contractions of more than 64 16-bit channels (shorter ones read W's own
 * layout with transposing LDS reads).  map_is_subm != 0 says map is a
 * submanifold nbr (n_src == n_rows); it changes nothing in the result or the
 * launch (every map with K > 1 runs the loop that keeps two offsets of
 * gathered rows in flight).  Other arguments and errors as
 * spc_conv_fwd_fused.
 */
spc_status spc_conv_fwd_wt(spc_dtype dtype, const void* feats, int64_t n_src, int32_t cin,
                           const void* weight_t, int32_t K, int32_t cout, const float* bias,
                           const int32_t* map, int32_t map_is_subm, const int32_t* order, int64_t n_rows,
                           const void* residual, int32_t relu, void* out, hipStream_t stream);

/*
 * The forward over a strided map's output rows when their count is in device
 * memory (spc_build_kmap_async's n_out_dev): the sparse convolution of spconv
 * USAGE.md, "Sparse Convolution", out[o] = act(bias + residual[o] +
 * sum_k feats[map[o*K + k]] @ W[k]).  The grid covers row_cap rows (the map's
 * out_cap); rows at or past *n_rows_dev are not written, and a count above
 * row_cap (an overflowed map) writes nothing.  weight_t = 0: weight
 * [K, cin, cout] as spc_sparse_conv_fwd takes it; weight_t != 0: weight
 * [K, cout, cin] from spc_transpose_weight, as spc_conv_fwd_wt.  feats
 * [n_src, cin], map [row_cap, K], order (NULL ok) [row_cap], residual (NULL
 * ok; may be out) and out [row_cap, cout]; results equal spc_conv_fwd_fused /
 * spc_conv_fwd_wt with n_rows = M bit for bit.  Errors as spc_conv_fwd_fused.
 */
spc_status spc_conv_fwd_dev_rows(spc_dtype dtype, const void* feats, int64_t n_src, int32_t cin,
                                 const void* weight, int32_t weight_t, int32_t K, int32_t cout,
                                 const float* bias, const int32_t* map, const int32_t* order,
                                 int64_t row_cap, const int32_t* n_rows_dev, const void* residual,
                                 int32_t relu, void* out, hipStream_t stream);

/*
 * dinput (Hygon spconv-das README, "Public Interface Support": forward, dinput
 * and dfilter): din[i] = sum over (k, o) with map_fwd[k][o] = i of
 * dout[o] @ W[k]^T, computed output-stationary over the input rows:
 *   map_is_subm != 0: map is the submanifold nbr [n_in, K] (n_out == n_in); by
 *                     symmetry din[i] = sum_k dout[nbr[i*K + K-1-k]] @ W[k]^T.
 *   map_is_subm == 0: map is the strided nbr_in [n_in, K];
 *                     din[i] = sum_k dout[nbr_in[i*K + k]] @ W[k]^T.
 * K == 1 with map NULL is the per-voxel case (n_out == n_in).  order (NULL
 * ok) is the order of the map's rows (order for subm, order_in for strided).
 * dout [n_out, cout], weight [K, cin, cout], din [n_in, cin] (overwritten).
 */
spc_status spc_conv_bwd_input(spc_dtype dtype, const void* dout, int64_t n_out, int32_t cout,
                              const void* weight, int32_t K, int32_t cin,
                              const int32_t* map, int32_t map_is_subm, const int32_t* order,
                              int64_t n_in, void* din, hipStream_t stream);

/* Host only.  Workspace bytes spc_conv_bwd_filter needs. */
spc_status spc_conv_bwd_filter_workspace(int64_t n_in, int64_t n_out, int32_t cin, int32_t cout,
                                         int32_t K, int32_t want_dbias, size_t* bytes);

/*
 * dfilter (Hygon spconv-das README, "Public Interface Support": training
 * covers forward, dinput and dfilter in FP32, FP16 and BF16), the weight
 * derivative of the forward sum:
 *   dW[k] = sum over the pairs (i, o) of offset k of feats[i]^T dout[o],
 * fp32 [K, cin, cout] (overwritten), from the CSR pair lists of
 * spc_build_kmap (pair_in = input rows i, pair_out = output rows o; for the
 * inverse layer pass them exchanged).  dbias (NULL ok) = column sums of dout,
 * fp32 [cout].  feats [n_in, cin] and dout [n_out, cout] share dtype.
 * K == 1 with all pair pointers NULL pairs row i with row i (n_in == n_out).
 * ws: spc_conv_bwd_filter_workspace bytes, 16-byte aligned, scratch.
 * Reduction: fixed-size pair chunks per offset, each a partial in the
 * workspace, summed in a fixed order, so the result is run-to-run identical.
 * Errors as spc_sparse_conv_fwd, plus SPC_ERR_WORKSPACE for a short ws.
 */
spc_status spc_conv_bwd_filter(spc_dtype dtype, const void* feats, int64_t n_in, int32_t cin,
                               const void* dout, int64_t n_out, int32_t cout, int32_t K,
                               const int32_t* pair_ptr, const int32_t* pair_in,
                               const int32_t* pair_out, float* dw, float* dbias,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * spc_conv_bwd_filter without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving or
 * training loops, harnesses that forbid hipMalloc.  Same arguments (minus ws
 * and ws_bytes), result bit for bit, and errors as spc_conv_bwd_filter.  Its
 * scratch is one static device array of SPC_DFILTER_SCRATCH_BYTES per GPU,
 * which each GPU the library runs on holds until the process ends; a call
 * whose spc_conv_bwd_filter_workspace size exceeds it returns
 * SPC_ERR_UNSUPPORTED (128 x 128 channels with K = 27 and dbias fit).  The
 * call allocates nothing.  Every call on one GPU shares that GPU's array:
 * calls that overlap in time on the same GPU (on other streams, or from other
 * host threads) race and must be serialised by the caller.  Nothing in the
 * array needs to start at zero: a call writes every scratch byte it reads.
 */
#define SPC_DFILTER_SCRATCH_BYTES (36u << 20)
spc_status spc_conv_bwd_filter_noalloc(spc_dtype dtype, const void* feats, int64_t n_in, int32_t cin,
                                       const void* dout, int64_t n_out, int32_t cout, int32_t K,
                                       const int32_t* pair_ptr, const int32_t* pair_in,
                                       const int32_t* pair_out, float* dw, float* dbias, hipStream_t stream);

/*
 * Sparse max pooling, forward (SparseMaxPool3d, spconv USAGE.md layer table:
 * downsampling whose dense version is nn.MaxPool3d, on the kernel map of a
 * strided layer with the pool's kernel size, stride and padding):
 *   out[o][c]  = max over k with nbr_out[o*K + k] >= 0 of feats[nbr_out[o*K + k]][c]
 *   argk[o][c] = the smallest such k reaching that maximum (ties go to the
 *                first offset), 255 when row o has no input (out is then 0).
 * feats [n_in, C], nbr_out [n_out, K] (a strided spc_build_kmap's nbr), out
 * [n_out, C] in the features' dtype (exact: a copy of the winning value),
 * argk uint8 [n_out, C] (NULL ok; the backward needs it).  C a positive
 * multiple of 16, at most 512 (fp16/bf16) or 256 (fp32); 1 <= K <= 254.  NaN
 * inputs are outside the contract.
 * SPC_ERR_UNSUPPORTED / SPC_ERR_ARG as the convolutions.
 */
spc_status spc_sparse_maxpool_fwd(spc_dtype dtype, const void* feats, int64_t n_in, int32_t C,
                                  const int32_t* nbr_out, int32_t K, int64_t n_out, void* out,
                                  uint8_t* argk, hipStream_t stream);

/*
 * Sparse max pooling, backward: each output's gradient goes, per channel, to
 * the input that won the maximum,
 *   din[i][c] = sum over k with o = nbr_in[i*K + k] >= 0 and argk[o][c] == k of dout[o][c],
 * summed in fp32 in offset order and rounded once (input-stationary over the
 * same kernel map's nbr_in [n_in, K]; no atomics, run-to-run identical).
 * dout [n_out, C], argk from spc_sparse_maxpool_fwd, din [n_in, C] overwritten.
 */
spc_status spc_sparse_maxpool_bwd(spc_dtype dtype, const void* dout, int64_t n_out, int32_t C,
                                  const uint8_t* argk, const int32_t* nbr_in, int32_t K, int64_t n_in,
                                  void* din, hipStream_t stream);

/* Host only.  Workspace bytes spc_point_to_voxel needs. */
spc_status spc_point_to_voxel_workspace(int64_t n_points, int32_t n_features, int64_t max_voxels,
                                        int32_t max_points, size_t* bytes);

/*
 * Point cloud to voxels (spconv.pytorch.utils.PointToVoxel, spconv USAGE.md:
 * "spconv.pytorch.utils API Reference" and the PointToVoxel example).
 * points [n_points, n_features] fp32 with x, y, z first (3 <= n_features <= 64);
 * vsize_xyz[3] and range_xyz[6] = {x_min, y_min, z_min, x_max, y_max, z_max}
 * are HOST arrays.  The grid has round((max - min) / vsize) voxels per axis
 * (at most 2^32 - 1 cells); a point's voxel is floor((p - min) / vsize) in
 * fp32, and it is inside iff that is within the grid on every axis.
 * Voxels are numbered in order of their first point; each keeps its first
 * max_points points in point order; once max_voxels voxels exist, points of
 * further voxels are dropped.  Outputs, first *n_voxels rows valid:
 *   voxels      fp32 [max_voxels, max_points, n_features]: the stored points,
 *               then (empty_mean != 0) the mean of the voxel's stored points
 *               in every unused slot, else zeros;
 *   coords      int32 [max_voxels, 3], (z, y, x) voxel coordinates, no batch;
 *   num_points  int32 [max_voxels], points stored in each voxel;
 *   pc_voxel_id int32 [n_points] (NULL ok): the voxel holding each point, -1
 *               when it lies outside or found no room;
 *   *n_voxels   (host) the number of voxels.
 * ws: spc_point_to_voxel_workspace bytes, 16-byte aligned.  Synchronises the
 * stream once, to return *n_voxels; every result is run-to-run identical.
 */
spc_status spc_point_to_voxel(const float* points, int64_t n_points, int32_t n_features,
                              const float* vsize_xyz, const float* range_xyz, int64_t max_voxels,
                              int32_t max_points, int32_t empty_mean, float* voxels, int32_t* coords,
                              int32_t* num_points, int32_t* pc_voxel_id, int64_t* n_voxels,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Per-point features from per-voxel ones (spconv.pytorch.utils
 * gather_features_by_pc_voxel_id, same page): out[i] = seg_features[id[i]],
 * zeros where pc_voxel_id[i] is outside [0, n_voxels).  seg_features
 * [n_voxels, C], out [n_points, C], C a positive multiple of 16.
 */
spc_status spc_gather_by_voxel_id(spc_dtype dtype, const void* seg_features, int64_t n_voxels, int32_t C,
                                  const int32_t* pc_voxel_id, int64_t n_points, void* out,
                                  hipStream_t stream);

/*
 * Measurement support (not part of the convolution): the dense MFMA rate of
 * this part, against which the convolutions' roofline fractions are read.
 * Launches `blocks` workgroups of 4 waves; each wave runs independent
 * accumulator chains of v_mfma_f32_16x16x32_bf16 (shape 0, 8 chains) or
 * v_mfma_f32_32x32x16_bf16 (shape 1, 4 chains) for `iters` rounds on
 * register operands, with no memory traffic in the loop.  sink: device
 * float [blocks * 256], written once per thread.  *flop (host, NULL ok)
 * receives the FLOP the launch executes; the caller times it on `stream`.
 */
spc_status spc_calibrate_mfma(int32_t shape, int32_t blocks, int32_t iters, float* sink, double* flop,
                              hipStream_t stream);

/* Description of the last failure on the calling thread ("" if none). */
const char* spc_last_error(void);

/* Library version string. */
const char* spc_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPC_H */
