/*
 * hlofusion.h -- C ABI of the hero-fusion library for AMD Instinct MI355X
 * (gfx950).
 *
 * The library executes ONE HLO fusion on one GPU: an elementwise prologue over
 * N-d arrays whose memory order is given by minor_to_major layouts, feeding
 * one "hero" -- a plain loop, a transpose, or a reduce -- that decides how the
 * whole fusion is emitted (XLA:GPU Emitters, "Hero-based codegen").
 *
 * Life cycle:
 *   hf_fusion_create   validate the descriptor, plan it (partition the DAG,
 *                      compose index maps, pick the hero and its tiling),
 *                      generate HIP source for it, compile it for gfx950 and
 *                      load it on the current device.  All validation happens
 *                      here, on the host, before any GPU call.
 *   hf_fusion_launch   run it on a caller-supplied stream with caller-owned
 *                      buffers; asynchronous; no allocation, no
 *                      synchronisation.
 *   hf_fusion_destroy  wait for the device, then release what create
 *                      allocated.
 *
 * Conventions:
 *   - Every function has C linkage and takes plain pointers and sizes only.
 *   - Device buffers and streams belong to the caller.  Buffers are dense and
 *     stored exactly in the declared layout (strided views are not accepted).
 *   - Errors: every call returns an hf_status; hf_last_error() gives a
 *     message for the last failing call on the calling thread.
 *   - A fusion handle is immutable after create and bound to the device that
 *     was current at create.  Launches hold no state in the handle: one handle
 *     may be launched from several threads and on several streams at once, as
 *     long as the buffers each launch writes (its result and its workspace)
 *     are not in use by another launch in flight.  The fusion computation
 *     writes only into the buffers it is given (XLA:GPU Emitters, "Loop
 *     emitter": the entry function inserts its results into the result
 *     buffers it receives).
 */
#ifndef HLOFUSION_H
#define HLOFUSION_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HF_ABI_VERSION 4
#define HF_MAX_RANK 8
#define HF_MAX_OPERANDS 9               /* concatenate is variadic; dynamic_slice takes the
                                           operand and one start index per dim */
#define HF_MAX_ATTR (3 * HF_MAX_RANK)   /* pad: low, high and interior per dim */
#define HF_MAX_PARAMS 16
#define HF_MAX_NODES 256

typedef enum {
  HF_OK = 0,
  HF_ERR_INVALID = 1,      /* the descriptor or a launch argument breaks a rule */
  HF_ERR_UNSUPPORTED = 2,  /* valid, but outside what this library implements */
  HF_ERR_COMPILE = 3,      /* the generated kernel did not compile */
  HF_ERR_HIP = 4,          /* a HIP runtime call failed */
  HF_ERR_NOMEM = 5
} hf_status;

/* Element types (StableHLO Specification, "Types": element types).
 * HF_S4 and HF_U4 are the 4-bit integers si4 and ui4 (ranges [-8, 7] and
 * [0, 15]).  The pages give no memory packing for them; this library packs
 * two elements per byte in physical (linear) order, the element with the even
 * linear index in the low four bits, so an array of n elements occupies
 * ceil(n / 2) bytes (the last byte's high half unused, and written as zero,
 * when n is odd).  A 4-bit result is written only by the loop hero with an
 * even number of elements per lane along an even physically minor dim, so
 * that no two lanes share a byte; other 4-bit results are HF_ERR_UNSUPPORTED.
 * 4-bit arrays can be read by every hero. */
typedef enum {
  HF_F32 = 0,
  HF_BF16 = 1,
  HF_F16 = 2,
  HF_S8 = 3,
  HF_U8 = 4,
  HF_S32 = 5,
  HF_S4 = 6,
  HF_U4 = 7
} hf_dtype;

/* Ops.  Semantics are those of the StableHLO Specification ("Ops") and of
 * Operation semantics (XlaBuilder), one section each:
 *   HF_PARAMETER          Parameter: fusion input number `parameter_number`.
 *   HF_CONSTANT           constant: the scalar `constant`, broadcast over the
 *                         node's type and rounded to its element type.
 *   HF_LOG, HF_EXP, HF_TANH          log, exponential, tanh (IEEE-754).
 *   HF_NEGATE, HF_ABS                negate, abs.
 *   HF_ADD, HF_SUBTRACT, HF_MULTIPLY, HF_DIVIDE   IEEE-754 arithmetic.
 *   HF_MAXIMUM, HF_MINIMUM           IEEE-754 maximum / minimum.
 *   HF_CONVERT            convert: int->float and float->float round to
 *                         nearest even; float->int truncates.
 *   HF_BROADCAST_IN_DIM   broadcast_in_dim, attr = broadcast_dimensions.
 *   HF_RESHAPE            reshape (same position in lexicographic order).
 *   HF_TRANSPOSE          transpose, attr = permutation: result dim d is
 *                         operand dim attr[d].
 *   HF_UNIFORM_DEQUANTIZE real = scale * (q - zero_point) (StableHLO
 *                         Quantization; per-tensor or per-axis).
 *   HF_UNIFORM_QUANTIZE   q = clamp(round_half_even(real / scale) +
 *                         zero_point, storage_min, storage_max).
 *   HF_REDUCE             reduce over attr = dimensions with `reducer` and
 *                         `init_value`.  At most one per fusion (its hero);
 *                         only elementwise ops may follow it.
 *   HF_REVERSE            reverse, attr = dimensions: operand index
 *                         dim - 1 - i along each of them.
 *   HF_IOTA               iota, no operands, attr[0] = iota_dimension: the
 *                         index along that dim, in the element type.
 *   HF_PAD                pad, operands {operand, padding_value (rank 0)},
 *                         attr = edge_padding_low[rank], edge_padding_high[rank],
 *                         interior_padding[rank]: result[i] =
 *                         operand[(i - low) / (interior + 1)] where that is an
 *                         operand element, else padding_value.
 *   HF_CONCATENATE        concatenate, operands = inputs (1..HF_MAX_OPERANDS),
 *                         attr[0] = dimension.
 *   HF_SLICE              slice, attr = start_indices[rank], limit_indices[rank],
 *                         strides[rank] (the attribute names of "Programs"):
 *                         result[i] = operand[start + i * strides], with
 *                         0 <= start <= limit <= dim(operand), strides >= 1 and
 *                         dim(result) = ceil((limit - start) / strides).
 *   HF_DYNAMIC_SLICE      dynamic_slice, operands = {operand, start index of
 *                         dim 0, ..., of dim rank-1}, attr = slice_sizes[rank]:
 *                         result[i] = operand[clamp(0, start, dim(operand) -
 *                         slice_sizes) + i] (StableHLO Specification,
 *                         "dynamic_slice").  The start indices are rank-0
 *                         integer parameters or constants of one type; a
 *                         parameter is read on the device at every launch.
 * The elementwise ops (add ... abs) also take per-tensor quantized operands
 * and results of one baseline type: the operands are dequantized, the op runs
 * on the f32 values and its result is quantized to the result type (each op's
 * semantics for quantized types in the StableHLO Specification).
 */
typedef enum {
  HF_PARAMETER = 0,
  HF_CONSTANT = 1,
  HF_ADD = 2,
  HF_SUBTRACT = 3,
  HF_MULTIPLY = 4,
  HF_DIVIDE = 5,
  HF_MAXIMUM = 6,
  HF_MINIMUM = 7,
  HF_LOG = 8,
  HF_EXP = 9,
  HF_TANH = 10,
  HF_NEGATE = 11,
  HF_ABS = 12,
  HF_CONVERT = 13,
  HF_BROADCAST_IN_DIM = 14,
  HF_RESHAPE = 15,
  HF_TRANSPOSE = 16,
  HF_UNIFORM_DEQUANTIZE = 17,
  HF_UNIFORM_QUANTIZE = 18,
  HF_REDUCE = 19,
  HF_REVERSE = 20,
  HF_IOTA = 21,
  HF_PAD = 22,
  HF_CONCATENATE = 23,
  HF_SLICE = 24,
  HF_DYNAMIC_SLICE = 25
} hf_op;

/* HF_REDUCER_ARGMAX is the variadic max/argmax reduce of Operation semantics
 * ("Variadic Reduce"): operands {values, indices}, where indices must be an
 * s32 iota along the single reduced dimension; the result (s32) is the index
 * part of the tuple fold f(max, argmax, value, index) = value >= max ?
 * (value, index) : (max, argmax), started from (init_value, constant).  The
 * library folds in parallel and combines partial results by larger value,
 * then larger index: ties go to the last index, as in the sequential fold, and
 * NaN values are never selected.  The index init (`constant`, any s32 value)
 * is the result exactly where no element is >= init_value, as in the
 * sequential fold. */
typedef enum {
  HF_REDUCER_ADD = 0,
  HF_REDUCER_MAX = 1,
  HF_REDUCER_MIN = 2,
  HF_REDUCER_ARGMAX = 3
} hf_reducer;

/* Uniform quantization parameters of a quantized element type (StableHLO
 * Specification, "Types": QuantizedTensorElementType, constraints C1-C13;
 * StableHLO Quantization, "Per-tensor quantization", "Per-axis
 * quantization").  The expressed type is f32; the storage type is the
 * hf_type's dtype (HF_S8, HF_U8, HF_S4 or HF_U4).  All arrays are HOST pointers read during
 * hf_fusion_create only; the library keeps its own copies. */
typedef struct {
  int32_t quantization_dimension;  /* -1: per-tensor; else the sliced dim */
  int32_t n;                       /* pairs: 1 (per-tensor) or dim(qdim) */
  const float *scales;             /* n values, each finite and > 0 */
  const int32_t *zero_points;      /* n values, storage_min <= zp <= storage_max */
  int32_t has_storage_range;       /* 0: storage range = range of dtype */
  int32_t storage_min, storage_max;
} hf_quant;

/* An array type: element type, dims (ascending dimension numbers), layout
 * (Shapes and layout, "Minor-to-major dimension ordering"; the first entry is
 * the most minor, fastest-varying dim).  has_layout = 0 selects the default
 * layout {rank-1, ..., 0} ("Default minor-to-major ordering").  Layouts are
 * physical only for parameters and the root; other nodes are virtual. */
typedef struct {
  int32_t dtype;                          /* an hf_dtype value */
  int32_t rank;                           /* 0 .. HF_MAX_RANK */
  int64_t dims[HF_MAX_RANK];              /* >= 0; size 0 is valid */
  int32_t has_layout;
  int32_t minor_to_major[HF_MAX_RANK];
  const hf_quant *quant;                  /* NULL unless a quantized type */
} hf_type;

/* One node of the fusion computation.  Operands are indices of EARLIER nodes
 * (the array is in topological order). */
typedef struct {
  int32_t op;                   /* an hf_op value */
  int32_t n_operands;
  int32_t operands[HF_MAX_OPERANDS];
  hf_type type;                 /* result type, stated explicitly */
  int32_t parameter_number;     /* HF_PARAMETER */
  double constant;              /* HF_CONSTANT (an integer constant is rank 0 and
                                   serves only as a dynamic_slice start index) */
  int32_t n_attr;
  int64_t attr[HF_MAX_ATTR];    /* permutation | broadcast_dimensions | dimensions |
                                   iota_dimension | pad's low, high, interior |
                                   concatenate's dimension | slice's start, limit,
                                   strides | dynamic_slice's slice_sizes */
  int32_t reducer;              /* HF_REDUCE: an hf_reducer value */
  double init_value;            /* HF_REDUCE (for HF_REDUCER_ARGMAX: the value
                                   init; `constant` holds the index init) */
} hf_node;

typedef struct {
  int32_t abi_version;          /* HF_ABI_VERSION */
  int32_t n_nodes;              /* 1 .. HF_MAX_NODES */
  const hf_node *nodes;
  int32_t root;                 /* index of the root node */
  int32_t n_params;             /* parameters are numbered 0 .. n_params-1 */
} hf_fusion_desc;

typedef struct hf_fusion hf_fusion;

typedef enum {
  HF_HERO_LOOP = 0,
  HF_HERO_TRANSPOSE = 1,
  HF_HERO_ROW_REDUCE = 2,
  HF_HERO_COLUMN_REDUCE = 3
} hf_hero;

/* What the planner chose.  Bytes are ALGORITHMIC: every parameter and the
 * per-axis quantization arrays read once, the result written once. */
typedef struct {
  hf_hero hero;
  int32_t n_partitions;         /* subgraph functions (XLA:GPU Emitters, "Partitioning") */
  int32_t vector_elems;         /* elements per lane per streaming access */
  int32_t block_threads;
  int64_t grid_blocks;
  int32_t lds_bytes;
  int64_t workspace_bytes;
  int64_t algorithmic_bytes;
  int64_t elements;             /* output elements (loop, transpose) or reduced inputs */
  int64_t rows, cols;           /* the normalised physical problem */
  int32_t tile_rows, tile_cols; /* transpose tile / reduce segment shape */
} hf_plan_info;

/* flags for hf_fusion_create */
#define HF_CREATE_PLAN_ONLY 1u     /* validate and plan; no code, no GPU */
#define HF_CREATE_COMPILE_ONLY 2u  /* also generate and compile; no GPU */

/* Validate, plan, generate, compile and load.  The descriptor is the fusion
 * instruction's called computation: its parameters, the op DAG in topological
 * order and its root (XLA:GPU Emitters: a fusion is an instruction with
 * operands and a called computation, "kind=kLoop, calls=..."; "Hero-based
 * codegen" picks the emitter from it).  The library copies what it needs;
 * the descriptor and every host array it points to may be freed on return.
 * On success *out owns a handle to free with hf_fusion_destroy.  Errors: HF_ERR_INVALID for a descriptor
 * that breaks an op's constraints (message names the node), HF_ERR_UNSUPPORTED
 * for a valid fusion this library does not implement (among them a parameter
 * or result of 2 GiB or more, or any value of 2^31 elements or more: the
 * kernels index with 32-bit offsets), HF_ERR_COMPILE, HF_ERR_HIP.  Nothing is
 * left allocated on failure. */
hf_status hf_fusion_create(const hf_fusion_desc *desc, uint32_t flags, hf_fusion **out);

/* Copy the plan into *info. */
hf_status hf_fusion_plan(const hf_fusion *f, hf_plan_info *info);

/* Copy the generated HIP source (NUL-terminated) into buf if cap suffices;
 * *len receives the length without the NUL.  HF_ERR_INVALID if the handle
 * was created with HF_CREATE_PLAN_ONLY. */
hf_status hf_fusion_source(const hf_fusion *f, char *buf, size_t cap, size_t *len);

/* Run the fusion (XLA:GPU Emitters, "Loop emitter": the entry function takes
 * the parameters and the result buffers and writes its results only into
 * those).  params[i] is the DEVICE pointer of parameter i (dense, in its
 * declared layout, 16-byte aligned; numel * element size bytes, 4-bit types
 * packed as described at hf_dtype); result is the device pointer of the root
 * buffer (dense, root layout, 16-byte aligned, not overlapping any
 * parameter).  The same parameter pointer may be passed twice, as the pages'
 * ABI passes two tensors that share a buffer slice once (XLA:GPU Emitters,
 * the passes that merge pointers to the same slice).
 *
 * workspace is scratch memory for this launch only, owned by the caller: a
 * device buffer of at least hf_plan_info.workspace_bytes bytes, 16-byte
 * aligned, overlapping neither the result nor a parameter.  Its contents on
 * entry do not matter and are undefined afterwards.  It may be NULL when
 * workspace_bytes is 0 (every plan except a reduce whose reduced extent is
 * split into several segments: a column reduce over many rows, a row reduce
 * of a few long rows).  Two launches in flight at the same time need two
 * workspaces.
 *
 * stream is a hipStream_t (NULL = the null stream).  The launch is
 * asynchronous and allocates nothing; a fault inside the kernel surfaces at
 * the caller's next synchronisation.  Each buffer must be device memory of
 * the fusion's device (or managed memory) whose whole extent lies in one
 * allocation; host memory, pinned or not, is rejected.  Errors:
 * HF_ERR_INVALID (count, NULL, alignment, overlap, not device memory, extent
 * past its allocation, workspace missing or too small, plan-only handle,
 * wrong current device), HF_ERR_HIP. */
hf_status hf_fusion_launch(hf_fusion *f, const void *const *params, int32_t n_params,
                           void *result, void *workspace, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * launch as hf_fusion_launch, with the library's own scratch memory in place
 * of the caller's workspace.  It allocates nothing.  The scratch memory is a
 * device array of HF_SCRATCH_BYTES per GPU, set up by hf_fusion_create and
 * held until the process ends.  A fusion whose workspace_bytes exceeds
 * HF_SCRATCH_BYTES is rejected with HF_ERR_UNSUPPORTED.  Every call on one GPU
 * shares that GPU's scratch memory: calls whose launches overlap in time on
 * one GPU (other streams, other threads) race on it and give wrong results;
 * run them on one stream or use hf_fusion_launch with separate workspaces.
 * Other arguments and errors as for hf_fusion_launch. */
#define HF_SCRATCH_BYTES (16u << 20)
hf_status hf_fusion_launch_noalloc(hf_fusion *f, const void *const *params, int32_t n_params,
                                   void *result, void *stream);

/* Release the handle (NULL is allowed).  It first waits for all work on the
 * fusion's device (hipDeviceSynchronize), so launches still in flight finish
 * before their code object is unloaded.  A HIP graph that captured a launch
 * of the handle must not be replayed after it is destroyed.  If the wait
 * fails (for example while a stream capture forbids it), nothing is released
 * and HF_ERR_HIP is returned: the handle stays valid and may be destroyed
 * again later. */
hf_status hf_fusion_destroy(hf_fusion *f);

/* Message of the last failing call on this thread ("" if none). */
const char *hf_last_error(void);

int32_t hf_abi_version(void);

/* Host helper: linear index of a logical multi-index under a layout
 * (Shapes and layout, "Array indexing").  Returns -1 on invalid input. */
int64_t hf_linear_index(int32_t rank, const int64_t *dims, const int32_t *minor_to_major,
                        const int64_t *index);

#ifdef __cplusplus
}
#endif

#endif /* HLOFUSION_H */
