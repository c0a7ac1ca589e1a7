/*
 * llvq.h -- C ABI of the LLVQ (Leech-lattice vector quantization) decode library for
 * AMD Instinct MI355X (gfx950).
 *
 * The method (arXiv 2603.11021, "Leech Lattice Vector Quantization for Efficient LLM
 * Compression"; papernotes.org notes, 方法详解 / 整体框架 and 关键设计 1, 2, 4;
 * gist.science summary, Methodik / 3. Indexierungsschema and 4.
 * Dequantisierungskernel; gptget.net, 原文摘要): weight rows are cut into 24-long
 * blocks along the input channels; each block is stored as an integer index of a
 * point of the Leech lattice (union of shells 2..M), optionally with a scalar-quantised
 * gain.  The library turns indices back into lattice points (shell -> class -> Golay
 * codeword / sign pattern / lexicographic permutation rank, undone with integer
 * division and modulo) and, in the fused GEMV, dots them with the activations without
 * writing decoded weights to memory.  The pages state the problem as converting to
 * and from bitstrings without materialising the codebook, plus a fully parallel
 * dequantisation kernel: llvq_decode / llvq_decode_many and llvq_gemv (index -> vector,
 * fused with the product) and llvq_encode_ref / llvq_encode_wide (vector -> index).  The
 * quantiser calls (llvq_search, llvq_quantize, the spherical-GPTQ calls) produce packed
 * tensors from fp32 weights.
 *
 * Conventions fixed by this library (the pages leave them open):
 *   Lattice coordinates are integers, sqrt(8) times the standard ones; shell m is the
 *   set of points with x.x = 16 m (standard squared norm 2m).  Shape indices number
 *   the points of shells 2..M in shell order, then class order, then
 *   I_class = r + A * (s + 2^B * R) with r the codeword, s the sign pattern and R the
 *   lexicographic rank of the absolute values.
 *
 *   Packed weights: a flat little-endian bitstream of fields of f = shape_bits +
 *   gain_bits bits, one per block, row-major over (row, block); field j starts at bit
 *   f*j and holds  shape | gain << shape_bits.  A row of K columns has
 *   Kb = ceil(K/24) blocks; columns K..24*Kb-1 are padding (activations are taken as
 *   zero there).  The buffer must hold llvq_packed_bytes(desc) bytes: the fields
 *   rounded up to 16 bytes plus 16 bytes of slack that the kernels may read.
 *
 *   Reconstruction: SHAPEGAIN w_hat = G[g] * v / (4 sqrt(m)), G a per-tensor fp16 table
 *   of 2^gain_bits entries; EUCLID w_hat = s[row] * v with s a per-row fp16 scale.
 *
 * Memory and streams: every array argument of the compute calls is a device pointer
 * owned by the caller.  The calls validate their arguments on the host, enqueue work
 * on `stream` (a hipStream_t; NULL means the default stream) and return without
 * synchronising.  The library allocates no device memory; its tables are compiled into
 * the shared object.  Its only state, per GPU and filled on first use under a lock, is
 * the device's CU count and LDS size (which size the tiled kernels' grids) and the address
 * of llvq_quantize_noalloc's workspace array.  Calls are thread-safe (llvq_quantize_noalloc
 * excepted: see there).
 *
 * Errors: synchronous return codes (below) report invalid arguments and launch
 * failures; nothing is enqueued when a call returns an error.  Data errors found on
 * the device (a shape index >= the number of points in shells 2..M, a point that is not
 * in the lattice or not in shells 2..M) are counted: if `err_count` is not NULL the
 * kernels add the number of such blocks/points to *err_count (a device int32, not
 * cleared by the library).  Such a block decodes to the zero vector; such a point
 * ranks to UINT64_MAX.
 */
#ifndef LLVQ_H_
#define LLVQ_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  LLVQ_OK = 0,
  LLVQ_EINVAL = -1,        /* invalid argument (null pointer, bad size, bad descriptor) */
  LLVQ_EUNSUPPORTED = -2,  /* valid request this library does not implement            */
  LLVQ_EHIP = -3,          /* the HIP runtime reported an error at launch (see below)  */
  LLVQ_ETOOLARGE = -4      /* more blocks than llvq_quantize_noalloc's fixed workspace */
};
/* LLVQ_EHIP: after its launches an entry point reads (and so clears) the calling thread's
 * last HIP error, as hipGetLastError does.  An error left pending by an earlier HIP call
 * of the same thread is therefore reported by the next LLVQ call as LLVQ_EHIP; the call's
 * own launches have still been made. */

enum { LLVQ_MODE_EUCLID = 0, LLVQ_MODE_SHAPEGAIN = 1 };
enum { LLVQ_OUT_POINTS_I8 = 0, LLVQ_OUT_BF16 = 1 };
enum { LLVQ_X_F32 = 0, LLVQ_X_BF16 = 1 };
enum { LLVQ_SEARCH_ANGULAR = 0, LLVQ_SEARCH_EUCLID = 1 };

#define LLVQ_MAX_BATCH 16

/* Description of one packed weight tensor W_hat [rows][cols]. */
typedef struct {
  int32_t mode;        /* LLVQ_MODE_EUCLID or LLVQ_MODE_SHAPEGAIN                        */
  int32_t rows;        /* N >= 1: output features                                        */
  int32_t cols;        /* K >= 1: input features; Kb = ceil(K/24) blocks per row          */
  int32_t max_shell;   /* M in [2, 42]: shape indices cover shells 2..M                  */
  int32_t shape_bits;  /* 1..120, with the index count of shells 2..M <= 2^shape_bits     */
  int32_t gain_bits;   /* EUCLID: 0.  SHAPEGAIN: 1..8.  shape_bits + gain_bits <= 128     */
} llvq_desc;

/* Rates.  The 2-bit kernels cover M <= 10 with shape_bits <= 60 and fields of at most 64
 * bits (2 bits per weight: 44 shape + 4 gain bits, M = 10).  Other rates (LLVQ,
 * papernotes.org notes, 关键设计 2: the same index hierarchy at any shell radius) go to a
 * general decoder: M up to 42 and fields up to 128 bits, e.g. 46 + 2 or 47 + 1 bits at
 * M = 11 or 12, or 3 bits per weight as 68 + 4 bits at M = 42, where global indices pass
 * 2^64.  Such descriptors are taken by llvq_packed_bytes, llvq_decode, llvq_decode_many
 * (one launch per tensor) and llvq_gemv.  The quantiser (llvq_search, llvq_quantize,
 * llvq_quantize_workspace_bytes) covers M <= 13 with fields of at most 64 bits (2 bits
 * per weight with 46..48 shape bits), the rank (llvq_encode_ref) M <= 33 (indices below
 * 2^64); past those, and for llvq_pack_fields past M = 10 or 64-bit fields, the calls
 * return LLVQ_EUNSUPPORTED (llvq_search and llvq_encode_ref, which take M directly,
 * LLVQ_EINVAL). */

/* Number of valid shape indices for shells 2..max_shell (|Lambda24(M)|).  Host only.
 * Writes *out and returns LLVQ_OK, or LLVQ_EINVAL if max_shell is outside [2, 10] or out
 * is NULL. */
int llvq_index_count(int32_t max_shell, uint64_t* out);

/* The same for M in [2, 42] as a 128-bit number (*lo | *hi << 64): past shell 33 the count
 * exceeds 64 bits (shell 42: just below 2^68).  Host only.  LLVQ_EINVAL for M outside
 * [2, 42] or a NULL output. */
int llvq_index_count_wide(int32_t max_shell, uint64_t* lo, uint64_t* hi);

/* Bytes the packed buffer of `d` must hold (see "Packed weights"), or a negative error
 * code for an invalid descriptor.  Host only. */
int64_t llvq_packed_bytes(const llvq_desc* d);

/* Static text for a return code.  Host only. */
const char* llvq_error_string(int code);

/* Decode every block of a packed tensor (gist.science, Methodik / 4.
 * Dequantisierungskernel: the index -> vector walk back through shell, class and the
 * local symmetries).
 *   packed  : llvq_packed_bytes(d) bytes, 16-byte aligned.
 *   scales  : fp16; SHAPEGAIN: gain table [2^gain_bits]; EUCLID: row scales [rows].
 *             Unused (may be NULL) for LLVQ_OUT_POINTS_I8.
 *   out_kind: LLVQ_OUT_POINTS_I8 -> out is int8 [rows][Kb*24], the raw integer lattice
 *             points including the padding columns (4-byte aligned);
 *             LLVQ_OUT_BF16 -> out is bf16 [rows][cols], the reconstructed weights with
 *             the padding columns dropped, each bit-defined as
 *             bf16_rne(f32(v) * f32(f32(G[g]) * f32(1/(4 sqrt m)))) (SHAPEGAIN) or
 *             bf16_rne(f32(v) * f32(s[row])) (EUCLID) (2-byte aligned).
 * Returns LLVQ_OK, LLVQ_EINVAL or LLVQ_EHIP. */
int llvq_decode(const llvq_desc* d, const void* packed, const void* scales, int32_t out_kind,
                void* out, int32_t* err_count, void* stream);

/* Decode several tensors in one call: the same result as llvq_decode on each, in one
 * launch when their tiles fit (one set-up, and the workgroups' stores spread over the
 * decode of other tiles instead of arriving together), else tensor by tensor.
 *   descs     : n descriptors (host array) with equal mode, max_shell, shape_bits and
 *               gain_bits; shapes may differ.
 *   n         : 1..16.
 *   packed    : host array of n device pointers (16-byte aligned), as for llvq_decode.
 *   scales    : host array of n device pointers (required for LLVQ_OUT_BF16, else may be
 *               NULL), as for llvq_decode.
 *   out_kind  : LLVQ_OUT_POINTS_I8 or LLVQ_OUT_BF16, for every tensor.
 *   outs      : host array of n device pointers, each laid out as llvq_decode's output.
 *   err_count : nullable; invalid indices of all tensors are counted together.
 * Returns LLVQ_OK, LLVQ_EINVAL (also for tensors that differ in widths or shell range) or
 * LLVQ_EHIP. */
int llvq_decode_many(const llvq_desc* descs, int32_t n, const void* const* packed, const void* const* scales,
                     int32_t out_kind, void* const* outs, int32_t* err_count, void* stream);

/* Fused dequantise-GEMV / small-batch GEMM: y[b][r] = sum_k W_hat[r][k] * x[b][k]
 * (papernotes.org, 关键设计 4: decode each block from its index and accumulate its dot
 * product with the activations without writing W_hat to memory).
 *   packed, scales : as for llvq_decode (scales required).
 *   x      : [batch][cols], contiguous, fp32 (LLVQ_X_F32, 4-byte aligned) or bf16
 *            (LLVQ_X_BF16, 2-byte aligned).
 *   batch  : 1..LLVQ_MAX_BATCH.
 *   y      : fp32 [batch][rows], 4-byte aligned, overwritten (never accumulated into).
 * Accumulation is fp32; results are deterministic (bitwise identical across runs).
 * Returns LLVQ_OK, LLVQ_EINVAL or LLVQ_EHIP. */
int llvq_gemv(const llvq_desc* d, const void* packed, const void* scales, const void* x,
              int32_t x_dtype, int32_t batch, float* y, int32_t* err_count, void* stream);

/* Rank lattice points: the inverse of the decode (gptget.net, 原文摘要: conversion to
 * and from bitstrings without materialising the codebook).
 *   points    : int8 [n][24] integer lattice coordinates (any alignment).
 *   n         : number of points, >= 0 (0 is a no-op).
 *   max_shell : M in [2, 33] (shells past 10 take a general rank kernel).
 *   indices   : uint64 [n] output shape indices (8-byte aligned); UINT64_MAX for a point
 *               that is not in the lattice or not in shells 2..M (counted in err_count).
 * Returns LLVQ_OK, LLVQ_EINVAL or LLVQ_EHIP. */
int llvq_encode_ref(const int8_t* points, int64_t n, int32_t max_shell, uint64_t* indices,
                    int32_t* err_count, void* stream);

/* The same with 128-bit indices, for shells up to 42 (past shell 33 indices exceed 64 bits;
 * 3 bits per weight is shell 42).
 *   points    : int8 [n][24], any alignment.
 *   max_shell : M in [2, 42].
 *   indices   : uint64 [n][2] output (8-byte aligned): index i is indices[2i] | indices[2i+1] << 64;
 *               both words all ones for a point that is not in the lattice or not in shells
 *               2..M (counted in err_count).
 * Returns LLVQ_OK, LLVQ_EINVAL or LLVQ_EHIP. */
int llvq_encode_wide(const int8_t* points, int64_t n, int32_t max_shell, uint64_t* indices,
                     int32_t* err_count, void* stream);

/* Quantise: nearest point of the shell union 2..M to each 24-vector, and its index
 * (papernotes.org notes, 关键设计 1: the single-shell search extended to the union of
 * shells 2..M, with an angular objective for shape-gain and a Euclidean one for spherical
 * shaping; gist.science page, Methodik / 2. Multi-Shell Search).  Exhaustive over every
 * class and every Golay codeword it can use, so the result is the exact optimum up to
 * fp32 rounding of the objective.
 *   x         : fp32 [n][24] input vectors, 4-byte aligned.  EUCLID takes them in the
 *               lattice's integer units (sqrt(8) x standard coordinates, shell m has
 *               squared norm 16 m).
 *   n         : number of vectors, >= 0 (0 is a no-op).
 *   max_shell : M in [2, 13].
 *   objective : LLVQ_SEARCH_ANGULAR maximises <x, v> / |v| (scale-free: collinear points
 *               of different shells tie, and the point of the lower shell is returned:
 *               u rather than 2u); LLVQ_SEARCH_EUCLID minimises |x - v|^2.
 *   points    : int8 [n][24] output, the chosen points (any alignment; also the input of
 *               the rank step that follows on the same stream).
 *   indices   : uint64 [n] output, the points' shape indices (8-byte aligned).
 *   err_count : nullable; a vector with a non-finite coordinate gets the
 *               zero point and index UINT64_MAX and is counted.
 * Exact float ties of the objective go to a fixed candidate order (not necessarily the
 * smaller index).  Both outputs are written on `stream`; the call allocates nothing.
 * Returns LLVQ_OK, LLVQ_EINVAL or LLVQ_EHIP. */
int llvq_search(const float* x, int64_t n, int32_t max_shell, int32_t objective, int8_t* points,
                uint64_t* indices, int32_t* err_count, void* stream);

/* Bytes of device workspace llvq_quantize needs for descriptor d (24 + 8 bytes per block,
 * the chosen points and their indices), or a negative LLVQ_* code for a bad descriptor. */
int64_t llvq_quantize_workspace_bytes(const llvq_desc* d);

/* Quantise a weight matrix into the packed stream that llvq_decode / llvq_gemv read: each
 * 24-block (zero-padded past the last column) gets its nearest point of shells 2..M and
 * the block's field is written (papernotes.org notes, 整体框架 and 关键设计 1: shape-gain
 * puts the block's direction on the lattice with the angular objective and scalar-quantises
 * the gain; spherical shaping takes the Euclidean nearest point; gist.science page,
 * Methodik / 2. Multi-Shell Search).
 *   d         : descriptor of the output tensor (as for llvq_decode).
 *   w         : fp32 [rows][cols] weights, 4-byte aligned.
 *   scales    : fp16, 2-byte aligned.  SHAPEGAIN: the gain table [2^gain_bits]; the block's
 *               shape is its angular nearest point and its gain index the nearest table
 *               entry to the block's norm (ties to the lower index).  EUCLID: per-row scales
 *               [rows]; the block divided by its row's scale (the lattice's integer units)
 *               gets its Euclidean nearest point.
 *   packed    : output stream of llvq_packed_bytes(d) bytes (16-byte aligned), every byte
 *               written (fields, then zero padding).
 *   workspace : llvq_quantize_workspace_bytes(d) bytes of device memory (8-byte aligned),
 *               owned by the caller; its contents are not meaningful after the call.
 *   err_count : nullable; a block with a non-finite value (after the row scale) is written
 *               with the all-ones shape field, which decodes to the zero block and is
 *               counted again by llvq_decode.
 * Exact ties of the search objective resolve as in llvq_search.  Runs on `stream`; the
 * call allocates nothing.  Returns LLVQ_OK, LLVQ_EINVAL or LLVQ_EHIP. */
int llvq_quantize(const llvq_desc* d, const float* w, const void* scales, void* packed, void* workspace,
                  int32_t* err_count, void* stream);

/* Spherical GPTQ (papernotes.org notes, 关键设计 3): quantisation with the layer Hessian's
 * error feedback, the block's lattice direction rescaled to the block's own norm (a
 * retraction onto the product of spheres) and its residual spread over the columns not yet
 * quantised through U = chol(H^-1)^T.  A caller runs, for a weight matrix W [rows][cols]:
 *   llvq_gptq_factor once, llvq_gptq_begin once, then for b = 0 .. Kb-1: llvq_search of the
 *   block column x (angular, shells 2..M) and llvq_gptq_column(b); finally llvq_pack_fields.
 * All matrices are fp64 on the device, row-major; Kp = 24 * Kb (cols rounded up to a whole
 * block); the calls allocate nothing and run on `stream`.
 *
 * Workspace bytes llvq_gptq_factor needs for `cols` columns (Kp*Kp*8 + Kb*576*8 + 256), or
 * LLVQ_EINVAL.  Host only. */
int64_t llvq_gptq_workspace_bytes(int32_t cols);

/* U [Kp][Kp] (upper triangular) with Hd^-1 = U^T U, Hd = Hp + damp * mean(diag H) * I, Hp =
 * H [cols][cols] padded to Kp with an uncoupled diagonal equal to mean(diag H) (pad columns
 * stay zero).  Computed without inverting Hd: with P the index reversal, P Hd P = M M^T
 * (Cholesky, blocked by 24) and U = P M^-1 P (blocked triangular inverse).
 *   H         : fp64 [cols][cols], symmetric positive (semi)definite.
 *   workspace : llvq_gptq_workspace_bytes(cols) bytes, 8-byte aligned, contents not kept.
 *   err_count : nullable; counts non-positive pivots (Hd not positive definite: U is then
 *               not meaningful).
 * Returns LLVQ_OK, LLVQ_EINVAL (null / misaligned pointer, cols <= 0, damp < 0) or LLVQ_EHIP. */
int llvq_gptq_factor(int32_t cols, const double* H, double damp, double* U, void* workspace,
                     int32_t* err_count, void* stream);

/* Wq [rows][Kp] fp64 = W [rows][cols] fp32 zero-padded, and x0 [rows][24] fp32 = the first
 * block column (the first search's input).  Returns LLVQ_OK, LLVQ_EINVAL or LLVQ_EHIP. */
int llvq_gptq_begin(int32_t rows, int32_t cols, const float* W, double* Wq, float* x0, void* stream);

/* One block column b after its search: for every row, the gain index nearest to the block's
 * norm (ties to the lower index), the field indices[r] | gain << shape_bits into
 * fields[r * Kb + b], the residual E = w - len v/|v| with len = |w| (variant 0, spherical)
 * or G[gain] (variant 1, Euclidean feedback), E' = E U_SS^-1, and W[:, F] -= E' U_SF for the
 * columns F after the block (variant 2, direct: no feedback); x_next [rows][24] fp32 receives
 * block column b + 1 (not written for the last block).
 *   d       : SHAPEGAIN descriptor (rows, cols, max_shell <= 13, shape_bits + gain_bits <= 64).
 *   gains   : fp16 [2^gain_bits].   points, indices: llvq_search's output for block b.
 *   ework   : fp64 [rows][24] scratch (may be NULL for variant 2).
 * Returns LLVQ_OK, LLVQ_EINVAL, LLVQ_EUNSUPPORTED or LLVQ_EHIP. */
int llvq_gptq_column(const llvq_desc* d, int32_t block, int32_t variant, const void* gains, double* Wq,
                     const double* U, const int8_t* points, const uint64_t* indices, uint64_t* fields,
                     double* ework, float* x_next, void* stream);

/* Invariant checks inside the kernels (a library built with LLVQ_DEVICE_CHECKS, for tests):
 * class and table indices in range, a positive count for every chosen value slot, queue
 * and ring capacities, codeword index below A.  A failed check adds one to a device
 * counter; nothing traps.  Writes the counter to *failures (host memory) and clears it when
 * reset != 0; synchronises with the device (it copies from a device symbol).  Returns
 * LLVQ_OK, LLVQ_EINVAL (failures NULL), LLVQ_EHIP, or LLVQ_EUNSUPPORTED in a library built
 * without the checks. */
int llvq_device_checks(uint32_t* failures, int32_t reset);

/* llvq_quantize for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels and the
 * same output, with the workspace held by the library instead of passed in.
 *   d, w, scales, packed, err_count, stream : as for llvq_quantize.
 * The workspace is a file-scope device array of llvq_quantize_noalloc_max_blocks() x 32
 * bytes (2^21 blocks, 64 MiB) that every GPU the library runs on holds until the process
 * ends; its device address is looked up once per GPU (with that GPU current) on the first
 * call that uses it.  Nothing in it has to start at zero: each call writes what it reads.
 * All calls on one GPU share the array, so calls that overlap on one GPU (several streams
 * or host threads at once) race and give undefined streams; serialise them.
 * The call allocates nothing (no hipMalloc / hipFree, no allocating library routine).
 * Returns LLVQ_ETOOLARGE (before any launch) when rows * Kb exceeds the maximum, else as
 * llvq_quantize (LLVQ_EHIP also when the array's address cannot be obtained). */
int llvq_quantize_noalloc(const llvq_desc* d, const float* w, const void* scales, void* packed,
                          int32_t* err_count, void* stream);

/* The most blocks (rows * Kb) llvq_quantize_noalloc accepts.  Host only. */
int64_t llvq_quantize_noalloc_max_blocks(void);

/* Write finished fields as the packed stream (the layout of llvq_decode's input): for
 * quantisers that choose the indices themselves (e.g. with error feedback between blocks).
 *   fields : uint64 [rows * Kb], field of block (r, b) at r * Kb + b, = shape index |
 *            gain index << shape_bits; bits above shape_bits + gain_bits are ignored
 *            (8-byte aligned).
 *   packed : llvq_packed_bytes(d) bytes (16-byte aligned), every byte written.
 * Returns LLVQ_OK, LLVQ_EINVAL or LLVQ_EHIP. */
int llvq_pack_fields(const llvq_desc* d, const uint64_t* fields, void* packed, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LLVQ_H_ */
