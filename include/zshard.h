/* zshard.h -- C ABI of libzshard: the per-shard optimizer step of ZeRO
 * stages 1/2/3 on one MI355X (gfx950) GPU.
 *
 * Pages cited (by title):
 *   [DP-III] 深度学习专题：模型训练的数据并行（三）
 *   [ZP]     ZeRO 原理：把模型状态切到多张 GPU 上
 *   [ZA]     ZeRO 技术原理：进阶与 Offload
 *   [EAI19]  高效AI 第19讲：分布式训练（第一部分）
 *
 * What rank k of P computes for its shard [s_k, e_k) of N parameters:
 *   g     = (sum over ranks r = 0..P-1, in that order, of grad_r[j]) / P   (fp32)
 *   m, v  = Adam moments of g, bias-corrected (standard or page-1 literal)
 *   w     = w - lr * m_hat / (sqrt(v_hat) + eps)                          (fp32)
 *   param[j] = w rounded to nearest-even fp16/bf16
 * for every global index j in [s_k, e_k).  Rows: [DP-III] §(三) 1. 步骤分析
 * (shard bounds), §(四) ZeRO-2 steps 2-4 (reduce-scatter, moments, update),
 * §(一) (Adam equations); [EAI19] 通信原语 All-Reduce (mean); [ZP] 核心原理
 * and [ZA] §2.2 (fp32 update, then the fp16 working copy: "float2half").
 *
 * Conventions for every entry point:
 *  - All device memory is owned by the caller.  The library allocates and
 *    frees nothing and keeps no state between calls other than a cached
 *    compute-unit count per device and a thread-local last HIP error.
 *    ([DP-III] §(五) ZeRO-R and [ZA] §1.4: fixed, pre-created buffers.)
 *  - Device pointers are plain HIP device addresses.  Arrays of pointers
 *    (`grads`) and all descriptor structs are host memory, read during the
 *    call only.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  Argument errors are returned synchronously, before anything is
 *    launched, and leave every buffer untouched.  A failed launch returns
 *    ZS_ERR_HIP (zs_last_hip_error() gives the hipError_t).  A fault inside a
 *    kernel surfaces at the caller's next synchronisation, as in any HIP code.
 *  - Shards that are empty (s_k == e_k) return ZS_OK without launching.
 *  - No alignment is required.  Arrays whose addresses line up on 16 bytes
 *    at a common element take the widest loads.
 *  - The functions are re-entrant; concurrent calls on one stream run in
 *    order, calls on different streams must not write the same memory.
 *  - Numerics: every fp32 constant is computed in double and rounded once;
 *    the mean is an fp32 left fold in rank order; no operation is fused
 *    (no FMA contraction); division and square root are correctly rounded;
 *    denormals are kept; NaN and inf propagate by IEEE rules.
 */
#ifndef ZSHARD_H
#define ZSHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZS_VERSION 1
#define ZS_MAX_P 256 /* ranks per step: the P gradient pointers travel as kernel arguments */

typedef enum {
  ZS_OK = 0,
  ZS_ERR_NULL = 1,     /* a required pointer is NULL */
  ZS_ERR_ARG = 2,      /* p, k, n, step, betas, lr, eps or form out of range */
  ZS_ERR_DTYPE = 3,    /* unknown dtype */
  ZS_ERR_RANGE = 4,    /* a base index lies past the shard start, or a size overflows */
  ZS_ERR_ALIAS = 5,    /* an output range overlaps another input or output range */
  ZS_ERR_CAPACITY = 6, /* a caller-provided table or workspace is too small */
  ZS_ERR_HIP = 7,      /* a HIP call failed; see zs_last_hip_error() */
  ZS_ERR_UNSUPPORTED = 8 /* the host CPU lacks an instruction set the call needs */
} zs_status;

typedef enum { ZS_F16 = 1, ZS_BF16 = 2 } zs_dtype;

/* Standard Adam stores the raw moving averages and bias-corrects them at use
 * ([ZA] §1.1.1; Kingma & Ba, its ref. 10).  The page-1 literal form stores
 * the corrected moments m_{t+1} = (b1 m_t + (1-b1) g)/(1 - b1^{t+1}) and
 * likewise v ([DP-III] §(一)); it is not equivalent to standard Adam. */
/* The update applied after the rank mean g.  The two Adam forms read and
 * write w, m, v; the SGD forms leave the state they do not use untouched, and
 * its pointers may then be NULL (m and v for ZS_SGD, v for ZS_SGD_MOMENTUM).
 *  ZS_SGD:          w = w - lr*g  ([DP-III] §(一), the SGD update); 2P + 10
 *                   bytes per element instead of 2P + 26.
 *  ZS_SGD_MOMENTUM: m = beta1*m + g; w = w - lr*m.  [ZA] §1.1.1 names SGD
 *                   with momentum and its stored buffer without a formula:
 *                   this is the heavy-ball form, coefficient beta1; 2P + 18
 *                   bytes per element.
 * beta2 and eps are validated but unused by the SGD forms. */
typedef enum {
  ZS_ADAM_STANDARD = 0,
  ZS_ADAM_PAGE1_LITERAL = 1,
  ZS_SGD = 2,
  ZS_SGD_MOMENTUM = 3
} zs_adam_form;

typedef struct {
  double lr;     /* learning rate, finite */
  double beta1;  /* in [0, 1) */
  double beta2;  /* in [0, 1) */
  double eps;    /* finite; added outside the square root ([DP-III] §(一) update eq.) */
  int64_t step;  /* t >= 1: the 1-based step being produced (bias corrections use beta^t) */
  int32_t form;  /* zs_adam_form */
  int32_t reserved; /* must be 0 */
} zs_adam_hparams;

/* Status name, e.g. "ZS_ERR_ARG". Never NULL. */
const char* zs_status_string(int32_t status);
/* ZS_VERSION of the built library. */
int32_t zs_version(void);
/* hipError_t of the last ZS_ERR_HIP on this thread (0 if none). */
int32_t zs_last_hip_error(void);

/* Shard plan ([DP-III] §(三) 1. 步骤分析): M = ceil(n/p); rank k owns
 * [min(kM, n), min((k+1)M, n)) (0-based, half-open; the page's 1-based
 * s_k = 1+(k-1)M, e_k = kM with both ends clamped to n).
 * n >= 0, 1 <= p (no upper limit here).  m_out, starts[p], ends[p] may each
 * be NULL.  Host-only: touches no device. */
zs_status zs_plan_shards(int64_t n, int32_t p, int64_t* m_out, int64_t* starts, int64_t* ends);

/* Arguments of the fused per-shard step.
 *  grads[r] (r = 0..p-1): rank r's gradient; grads[r][i] holds global index
 *     grad_base + i.  grad_base = 0 for full-length buffers, = s_k for buffers
 *     that hold only this shard.  Read only.  dtype grad_dtype.
 *  w, m, v: fp32, e_k - s_k elements each, element i = global s_k + i,
 *     updated in place.  m0 = v0 = 0 at step 1 ([DP-III] §(一)).  m and v
 *     may be NULL for a form that does not use them (see zs_adam_form).
 *  param: the 16-bit working copy; param[j - param_base] is written for each
 *     j in [s_k, e_k) and nothing else.  param_base = 0 for a full-length
 *     working copy (this rank's contribution to the all-gather).
 *  The library computes s_k and e_k from (n, p, k) itself. */
typedef struct {
  int64_t n;                 /* parameters N >= 0 */
  int32_t p;                 /* ranks, 1..ZS_MAX_P */
  int32_t k;                 /* this rank, 0..p-1 */
  const void* const* grads;  /* host array of p device pointers, rank order */
  int32_t grad_dtype;        /* zs_dtype */
  int32_t param_dtype;       /* zs_dtype */
  int64_t grad_base;         /* 0 <= grad_base <= s_k */
  float* w;
  float* m;
  float* v;
  void* param;
  int64_t param_base;        /* 0 <= param_base <= s_k */
  const zs_adam_hparams* hp;
  void* stream;              /* hipStream_t */
} zs_shard_args;

/* The whole step in one kernel: gather + rank-order mean + Adam + downcast.
 * Memory traffic per element (Adam): 2p (grads) + 12 (w, m, v read) + 12
 * (write) + 2 (param) bytes; 2p + 10 for ZS_SGD, 2p + 18 for
 * ZS_SGD_MOMENTUM.  The fp32 mean is never stored ([DP-III] §(三) step 4:
 * the gradient is released after the update).
 * Errors: ZS_ERR_NULL (args, hp, grads, any grads[r], w, param, or m / v
 * when the form uses them, when the shard is non-empty), ZS_ERR_ARG,
 * ZS_ERR_DTYPE, ZS_ERR_RANGE, ZS_ERR_ALIAS (the buffers the form writes
 * overlap each other or any gradient range), ZS_ERR_HIP. */
zs_status zs_fused_shard_step(const zs_shard_args* args);

/* The gradient mean alone, stored (the local stand-in for reduce-scatter +
 * mean; [DP-III] §(四) step 2 keeps the slice mean in memory before the
 * moment update): g_out[i] = mean over ranks of global
 * index s_k + i, for i in [0, e_k - s_k).  g_out: fp32 device array.
 * grads / grad_dtype / grad_base as in zs_shard_args.  Traffic 2p + 4 B/elem. */
zs_status zs_reduce_scatter_mean_local(const void* const* grads, int32_t grad_dtype,
                                       int64_t grad_base, int64_t n, int32_t p, int32_t k,
                                       float* g_out, void* stream);

/* Adam + downcast from a stored fp32 gradient (the unfused second half):
 * len elements of g (read), w, m, v (updated) and param (written,
 * param_dtype).  param may be NULL to skip the downcast.  Traffic 30 B/elem
 * (28 without param). */
zs_status zs_adam_step(const float* g, float* w, float* m, float* v, void* param,
                       int32_t param_dtype, int64_t len, const zs_adam_hparams* hp,
                       void* stream);

/* ---- many tensors in one launch ------------------------------------------
 * A shard of a flattened parameter list meets several tensors.  Each
 * intersection is a piece; pieces are cut into chunks of at most
 * chunk_elems elements, and one persistent launch walks the chunk table
 * (the analogue of gradient buckets, [ZA] §1.4 ZeRO-R and §1.5).  One
 * workgroup per CU takes one chunk at a time, so the chunk is the unit of
 * load balance.  A good chunk_elems is 57,344 (= 28 * 256 * 8, the kernel's
 * whole chunk).  For a shard under two of those per CU, use the shard
 * length divided by the CU count, rounded up to a multiple of 2,048, and a
 * quarter of that when the shard has several pieces (more chunks per CU even
 * things out where the pieces end). */
typedef struct {
  int32_t tensor;      /* index in the caller's tensor list */
  int32_t reserved;
  int64_t tensor_off;  /* first element of the piece inside that tensor */
  int64_t shard_off;   /* first element of the piece inside the shard [s_k, e_k) */
  int64_t len;         /* elements */
} zs_piece;

/* Pieces of rank k's shard over tensors of numel[0..ntensors) flattened in
 * list order.  Writes up to pieces_cap pieces, sets *npieces and, when
 * chunk_elems > 0 and nchunks_out is given, the chunk count.  Zero-size
 * tensors yield no piece.  ZS_ERR_CAPACITY if more than pieces_cap pieces
 * (then *npieces holds the count needed).  Host-only. */
zs_status zs_plan_chunks(const int64_t* numel, int32_t ntensors, int32_t p, int32_t k,
                         int64_t chunk_elems, zs_piece* pieces, int32_t pieces_cap,
                         int32_t* npieces, int64_t* nchunks_out);

/* Device pointers of one piece, each already at the piece's first element:
 * w/m/v fp32, param 16-bit, grads[r] the 16-bit gradient of rank r (host
 * array of p device pointers).  m and v may be NULL; a step whose form needs
 * them then fails with ZS_ERR_NULL unless every piece has them. */
typedef struct {
  float* w;
  float* m;
  float* v;
  void* param;
  const void* const* grads;
} zs_piece_ptrs;

/* Host-side handle of an uploaded launch table (filled by zs_mt_upload). */
typedef struct {
  const void* workspace; /* device memory holding the table */
  int64_t nchunks;
  int64_t chunk_elems;
  int32_t npieces;
  int32_t p;
  int32_t grad_dtype;
  int32_t param_dtype;
  int32_t state;    /* ZS_STATE_M | ZS_STATE_V: every piece has that buffer */
  int32_t reserved;
} zs_mt_table;

#define ZS_STATE_M 1
#define ZS_STATE_V 2

/* Bytes of device workspace that zs_mt_upload needs (0 on bad arguments). */
size_t zs_mt_workspace_bytes(int32_t npieces, int64_t nchunks, int32_t p);

/* Writes the launch table (piece descriptors, gradient pointers, chunk list)
 * into the caller's device workspace (>= zs_mt_workspace_bytes bytes,
 * 256-byte aligned) with one host-to-device copy on `stream`, waits for that
 * copy, and fills *table.  pieces[i].len and pieces[i].shard_off come from
 * zs_plan_chunks (or any list of disjoint pieces); ptrs[i] are the device
 * pointers at each piece's first element.  Call once per plan: the table
 * stays valid while the memory it points to does.
 * Errors: ZS_ERR_NULL, ZS_ERR_ARG (p outside 1..ZS_MAX_P, chunk_elems < 8 or
 * not a multiple of 8, npieces < 0, a piece len < 1), ZS_ERR_DTYPE,
 * ZS_ERR_CAPACITY (ws_bytes too small or workspace misaligned), ZS_ERR_ALIAS
 * (an output of one piece overlaps an output of any piece or a gradient
 * range), ZS_ERR_HIP. */
zs_status zs_mt_upload(const zs_piece* pieces, const zs_piece_ptrs* ptrs, int32_t npieces,
                       int32_t p, int32_t grad_dtype, int32_t param_dtype, int64_t chunk_elems,
                       void* workspace, size_t ws_bytes, void* stream, zs_mt_table* table);

/* The fused step over every chunk of an uploaded table in one persistent launch;
 * each block stages its chunk's descriptor and the p gradient pointers in
 * LDS.  Same arithmetic and traffic per element as zs_fused_shard_step.
 * A table with no chunks returns ZS_OK without launching.
 * Errors: ZS_ERR_NULL, ZS_ERR_ARG (hparams or a table field out of range),
 * ZS_ERR_DTYPE, ZS_ERR_HIP. */
zs_status zs_fused_shard_step_multi(const zs_mt_table* table, const zs_adam_hparams* hp,
                                    void* stream);

/* ---- optimizer offload: the update on the host CPU -----------------------
 * [ZA] §2.2 Offload 策略: the GPU sends the shard's 16-bit gradient to host
 * memory, the CPU keeps the fp32 master weights and moments and runs the
 * update and the float2half conversion, and the 16-bit parameters go back;
 * [ZA] §1.6.2: multithreaded SIMD, one CPU process per GPU shard.
 * All pointers are HOST memory.  g: len 16-bit gradients (grad_dtype), e.g.
 * the rank mean rounded to 16 bits on the GPU; w, m, v: fp32, updated in
 * place (m / v may be NULL when the form does not use them, as for
 * zs_fused_shard_step); param: len 16-bit outputs (param_dtype) or NULL.
 * Same per-element arithmetic as zs_adam_step applied to the widened
 * gradient, bit for bit, on 8 lanes at a time (AVX2 + F16C, no FMA), in
 * `threads` threads (<= 0: all hardware threads; at most one per 64 Ki
 * elements).  Synchronous; returns when done.  Traffic per element: 2 + 12
 * + 12 + 2 bytes for Adam (2 + 4 + 4 + 2 for SGD, 2 + 8 + 8 + 2 for momentum).
 * Errors: ZS_ERR_NULL, ZS_ERR_ARG, ZS_ERR_DTYPE, ZS_ERR_RANGE, ZS_ERR_ALIAS
 * (the buffers written overlap each other or g), ZS_ERR_UNSUPPORTED (no
 * AVX2/F16C on this CPU). */
zs_status zs_cpu_adam_step(const void* g, int32_t grad_dtype, float* w, float* m, float* v,
                           void* param, int32_t param_dtype, int64_t len,
                           const zs_adam_hparams* hp, int32_t threads);

#ifdef __cplusplus
}
#endif

#endif /* ZSHARD_H */
