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
 *    Host memory the call needs for its own bookkeeping that cannot be had
 *    gives ZS_ERR_RESOURCE (no exception crosses this interface).
 *  - Shards that are empty (s_k == e_k) return ZS_OK without launching.
 *  - No alignment is required.  The kernels run fastest when the arrays'
 *    element 0 sits on a 128-byte line (or all sit the same distance into
 *    one); the call peels 0-7 leading elements to line up as many of the
 *    arrays' bytes as it can.
 *  - The functions are re-entrant; concurrent calls on one stream run in
 *    order, calls on different streams must not write the same memory.
 *    The whole-chunk kernels pace their workgroups through small device
 *    counters shared by all calls on a GPU; calls overlapping on different
 *    streams may slow each other there, never change each other's
 *    results.
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

#define ZS_VERSION 2
#define ZS_MAX_P 1024 /* ranks per step */
/* Up to ZS_KERNARG_P ranks, a launch carries the gradient pointers in its
 * kernel arguments; the fused step with more ranks reads them from a
 * caller-owned device workspace (zs_shard_args.workspace). */
#define ZS_KERNARG_P 256

typedef enum {
  ZS_OK = 0,
  ZS_ERR_NULL = 1,     /* a required pointer is NULL */
  ZS_ERR_ARG = 2,      /* p, k, n, step, betas, lr, eps or form out of range */
  ZS_ERR_DTYPE = 3,    /* unknown dtype */
  ZS_ERR_RANGE = 4,    /* a base index lies past the shard start, or a size overflows */
  ZS_ERR_ALIAS = 5,    /* an output range overlaps another input or output range */
  ZS_ERR_CAPACITY = 6, /* a caller-provided table or workspace is too small */
  ZS_ERR_HIP = 7,      /* a HIP call failed; see zs_last_hip_error() */
  ZS_ERR_UNSUPPORTED = 8, /* the host CPU lacks an instruction set the call needs */
  ZS_ERR_RESOURCE = 9     /* host memory or a host thread could not be obtained */
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
  /* Device memory for the rank pointer table, used only when p >
   * ZS_KERNARG_P (may be NULL otherwise): at least zs_shard_workspace_bytes(p)
   * bytes, 16-byte aligned, overlapping no other buffer of the call.  Each
   * call rewrites it on `stream` before its step, so calls that share a
   * workspace must run on one stream. */
  void* workspace;
  size_t workspace_bytes;
} zs_shard_args;

/* Bytes of zs_shard_args.workspace needed for p ranks: 0 for p <=
 * ZS_KERNARG_P, else 8 * p rounded up to 256 (0 also for p outside
 * 1..ZS_MAX_P). */
size_t zs_shard_workspace_bytes(int32_t p);

/* The whole step in one kernel: gather + rank-order mean + Adam + downcast.
 * Memory traffic per element (Adam): 2p (grads) + 12 (w, m, v read) + 12
 * (write) + 2 (param) bytes; 2p + 10 for ZS_SGD, 2p + 18 for
 * ZS_SGD_MOMENTUM.  The fp32 mean is never stored ([DP-III] §(三) step 4:
 * the gradient is released after the update).  With p > ZS_KERNARG_P one
 * small launch per 256 ranks first writes the rank pointers into the
 * workspace.
 * Errors: ZS_ERR_NULL (args, hp, grads, any grads[r], w, param, or m / v
 * when the form uses them, when the shard is non-empty), ZS_ERR_ARG,
 * ZS_ERR_DTYPE, ZS_ERR_RANGE, ZS_ERR_ALIAS (the buffers the form writes, or
 * the workspace, overlap each other or any gradient range), ZS_ERR_CAPACITY
 * (p > ZS_KERNARG_P and the workspace is NULL, too small or not 16-byte
 * aligned), ZS_ERR_HIP. */
zs_status zs_fused_shard_step(const zs_shard_args* args);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * step as zs_fused_shard_step, bit for bit, with the rank pointer table of p
 * > ZS_KERNARG_P ranks kept in a static device array of the library
 * (ZS_STATIC_SCRATCH_BYTES per GPU, held until the process ends) instead of
 * args->workspace, which is ignored.  Allocates nothing: no hipMalloc, no
 * hipFree, no allocating library call.  Every call on one GPU shares that
 * GPU's array, so calls that overlap on one GPU (on different streams) race
 * and must not be issued; calls on one stream are ordered and safe.  For p <=
 * ZS_KERNARG_P it uses no scratch at all.  Errors: as zs_fused_shard_step,
 * ZS_ERR_CAPACITY if the table would exceed the array. */
#define ZS_STATIC_SCRATCH_BYTES 8192 /* ZS_MAX_P rank pointers */
zs_status zs_fused_shard_step_static(const zs_shard_args* args);

/* The gradient mean alone, stored (the local stand-in for reduce-scatter +
 * mean; [DP-III] §(四) step 2 keeps the slice mean in memory before the
 * moment update): g_out[i] = mean over ranks of global
 * index s_k + i, for i in [0, e_k - s_k).  g_out: fp32 device array.
 * grads / grad_dtype / grad_base as in zs_shard_args.  Traffic 2p + 4 B/elem.
 * With p > ZS_KERNARG_P the ranks go in passes of 256: each pass continues
 * the fp32 rank-order sums that the previous pass left in g_out (8 B/elem
 * more per extra pass), so the result is the same left fold.
 * Errors: ZS_ERR_NULL, ZS_ERR_ARG, ZS_ERR_DTYPE, ZS_ERR_RANGE, ZS_ERR_ALIAS
 * (g_out overlaps a gradient range), ZS_ERR_HIP. */
zs_status zs_reduce_scatter_mean_local(const void* const* grads, int32_t grad_dtype,
                                       int64_t grad_base, int64_t n, int32_t p, int32_t k,
                                       float* g_out, void* stream);

/* The same mean rounded to nearest even in 16 bits (out_dtype): the
 * "gradient 16" that the GPU hands to the CPU when the update is offloaded
 * ([ZA] §2.2 Offload 策略: the graph is cut along the fp16 gradient and fp16
 * parameter edges).  g_out: L_k 16-bit elements.  The mean is formed in
 * fp32 exactly as above and rounded once.  p > ZS_KERNARG_P also needs
 * `partial`: an fp32 device array of L_k elements for the sums between
 * passes (may be NULL otherwise).  Traffic 2p + 2 B/elem.
 * Errors: as zs_reduce_scatter_mean_local, plus ZS_ERR_NULL for a missing
 * `partial` and ZS_ERR_ALIAS if g_out or partial overlap a gradient range
 * or each other. */
zs_status zs_reduce_scatter_mean_local16(const void* const* grads, int32_t grad_dtype,
                                         int64_t grad_base, int64_t n, int32_t p, int32_t k,
                                         void* g_out, int32_t out_dtype, float* partial,
                                         void* stream);

/* Adam + downcast from a stored fp32 gradient (the unfused second half):
 * [DP-III] §(四) step 3 (moments of this shard from the stored slice mean)
 * and step 4 (the shard's parameters from the moments); the 16-bit copy as
 * in [ZA] §2.2 float2half.  len elements of g (read), w, m, v (updated) and
 * param (written, param_dtype).  param may be NULL to skip the downcast.
 * Traffic 30 B/elem (28 without param).
 * Errors: ZS_ERR_NULL, ZS_ERR_ARG, ZS_ERR_DTYPE, ZS_ERR_RANGE, ZS_ERR_ALIAS
 * (an output overlaps g or another output), ZS_ERR_HIP. */
zs_status zs_adam_step(const float* g, float* w, float* m, float* v, void* param,
                       int32_t param_dtype, int64_t len, const zs_adam_hparams* hp,
                       void* stream);

/* ---- many tensors in one launch ------------------------------------------
 * A shard of a flattened parameter list meets several tensors.  Each
 * intersection is a piece; pieces are cut into chunks of at most
 * chunk_elems elements, and one persistent launch walks the chunk table
 * (the analogue of gradient buckets: [ZA] §1.4 ZeRO-R keeps fixed,
 * pre-created buffers and moves small pieces of data bucketed together;
 * §1.5 reduces each 1/N of the gradient in buckets).  One workgroup per CU
 * takes one chunk at a time, so the chunk is the unit of load balance;
 * zs_mt_chunk_elems gives the chunk length to use. */
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

/* The chunk length for a shard (or bucket) of shard_len elements in npieces
 * tensor pieces on cu_count compute units (<= 0: the current device's):
 * 57,344 (= 28 * 256 * 8, the kernel's whole chunk) when the shard holds at
 * least two of those per CU; otherwise the shard's per-CU share, a quarter
 * of it when npieces > 1 (chunks end unevenly where pieces end, and more
 * chunks per CU even that out), rounded up to a multiple of 2,048.  0 on
 * bad arguments (shard_len < 0, npieces < 1).  Host-only, apart from the
 * device query when cu_count <= 0. */
int64_t zs_mt_chunk_elems(int64_t shard_len, int32_t npieces, int32_t cu_count);

/* Buckets of a shard ([ZA] §1.5: the shard's gradient is reduced bucket by
 * bucket as backward fills them; ZeRO-R's fixed buffers, §1.4): runs of
 * consecutive pieces, each closed as soon as it holds at least bucket_elems
 * elements (the last run may hold fewer).  bucket_of[i] receives the bucket
 * of piece i (0-based, non-decreasing), *nbuckets their count.
 * bucket_elems <= 0 puts every piece in bucket 0.  Host-only.
 * Errors: ZS_ERR_NULL, ZS_ERR_ARG (npieces < 0 or a piece len < 1). */
zs_status zs_plan_buckets(const zs_piece* pieces, int32_t npieces, int64_t bucket_elems,
                          int32_t* bucket_of, int32_t* nbuckets);

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

/* [ZA] §1.4 (ZeRO-R: a fixed buffer created once, not per step) and §1.5
 * (buckets): writes the launch table (piece descriptors, gradient pointers,
 * chunk list) into the caller's device workspace (>= zs_mt_workspace_bytes bytes,
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

/* The fused step over every chunk of an uploaded table in one persistent launch
 * (the per-shard step of [DP-III] §(四) steps 2-4 over a bucket or a whole
 * shard, [ZA] §1.5); each block stages its chunk's descriptor and the p
 * gradient pointers in LDS.  Same arithmetic and traffic per element as
 * zs_fused_shard_step.
 * A table with no chunks returns ZS_OK without launching.
 * Errors: ZS_ERR_NULL, ZS_ERR_ARG (hparams or a table field out of range),
 * ZS_ERR_DTYPE, ZS_ERR_HIP. */
zs_status zs_fused_shard_step_multi(const zs_mt_table* table, const zs_adam_hparams* hp,
                                    void* stream);

/* ---- step constants in device memory (launches captured once, replayed) --
 * A launch captured in a HIP graph replays its kernel arguments unchanged,
 * but Adam's bias corrections change every step (beta^t, [DP-III] §(一)).
 * A step table holds the fp32 constants of nsteps consecutive steps,
 * computed on the host exactly as for a by-value call (each in double,
 * rounded once), plus a cursor.  zs_fused_shard_step_multi_dev reads the
 * entry at the cursor on the device; zs_step_table_advance moves the cursor
 * with a one-thread kernel.  Captured as [bucket launches..., advance], a
 * graph replays consecutive steps: the bucketed update of [ZA] §1.5 with
 * the launch cost of one graph.  A launch that finds the cursor past the
 * last entry updates nothing and sets `exhausted`. */
typedef struct {
  void* dev;            /* device memory holding the table */
  int64_t first_step;   /* the step of entry 0 */
  int32_t nsteps;
  int32_t p;            /* ranks whose mean the entries divide by */
  int32_t form;         /* zs_adam_form of every entry */
  int32_t reserved;
} zs_step_table;

/* Entries of one step table at most (36 bytes each on the device, staged
 * once in host memory by zs_step_table_init). */
#define ZS_MAX_TABLE_STEPS (1 << 24)

/* Device bytes of a step table of nsteps entries (0 if nsteps is outside
 * 1..ZS_MAX_TABLE_STEPS). */
size_t zs_step_table_bytes(int32_t nsteps);

/* Fills a step table for steps hp->step .. hp->step + nsteps - 1 with hp's
 * lr, betas, eps and form, cursor 0, in the caller's device memory (>=
 * zs_step_table_bytes(nsteps) bytes, 256-byte aligned), with one
 * host-to-device copy on `stream`, and waits for it (not capturable; call it
 * before capture).  Errors: ZS_ERR_NULL, ZS_ERR_ARG (hparams, p outside
 * 1..ZS_MAX_P, nsteps outside 1..ZS_MAX_TABLE_STEPS), ZS_ERR_CAPACITY,
 * ZS_ERR_HIP, ZS_ERR_RESOURCE. */
zs_status zs_step_table_init(const zs_adam_hparams* hp, int32_t p, int32_t nsteps, void* dev,
                             size_t bytes, void* stream, zs_step_table* table);

/* cursor += 1, as a one-thread kernel on `stream` (capturable). */
zs_status zs_step_table_advance(const zs_step_table* table, void* stream);

/* Reads the cursor and the exhausted flag back to the host: one
 * device-to-host copy on `stream`, then waits for it. */
zs_status zs_step_table_status(const zs_step_table* table, int64_t* cursor, int32_t* exhausted,
                               void* stream);

/* zs_fused_shard_step_multi with the step constants read on the device from
 * the step table's current entry (capturable: nothing step-dependent is in
 * the kernel arguments).  The table's p and form must match: p of the chunk
 * table, and form's state (ZS_ERR_NULL if the chunk table lacks m or v that
 * the form needs). */
zs_status zs_fused_shard_step_multi_dev(const zs_mt_table* table, const zs_step_table* steps,
                                        void* stream);

/* ---- optimizer offload: the update on the host CPU -----------------------
 * [ZA] §2.2 Offload 策略: the GPU sends the shard's 16-bit gradient to host
 * memory, the CPU keeps the fp32 master weights and moments and runs the
 * update and the float2half conversion, and the 16-bit parameters go back;
 * [ZA] §1.6.2: multithreaded SIMD; §2.3 扩展性: one CPU process per GPU shard.
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

/* ---- optimizer offload on one GPU: the pipeline ------------------------
 * [ZA] §2.2 Offload 策略: the GPU forms the shard's gradient, rounds it to 16
 * bits and sends it to host memory bucket by bucket as the buckets fill (the
 * copies overlap the GPU's work); the CPU runs the update and float2half on
 * the fp32 state in host memory; the 16-bit parameters go back to the GPU's
 * working copy while the CPU updates the next bucket.
 * [ZA] §2.3 扩展性, delayed parameter update: steps 1..N-1 update normally
 * (ZS_OFFLOAD_PLAIN); at step N the CPU receives the gradient and does not
 * update (ZS_OFFLOAD_RECEIVE); from step N+1 on it applies the gradient
 * received the step before while this step's gradient is formed and received
 * (ZS_OFFLOAD_DELAYED).  The schedule, and the update count hp->step that
 * each applied gradient gets, are the caller's. */
typedef enum {
  ZS_OFFLOAD_PLAIN = 0,    /* receive this step's gradient into slot, update with it */
  ZS_OFFLOAD_RECEIVE = 1,  /* receive into slot only */
  ZS_OFFLOAD_DELAYED = 2   /* update with slot 1-slot (last step's) while receiving into slot */
} zs_offload_mode;

typedef struct {
  /* device side: as in zs_shard_args */
  int64_t n;
  int32_t p, k;
  const void* const* grads;  /* host array of p device pointers */
  int32_t grad_dtype;        /* also the dtype of the 16-bit gradient sent to the host */
  int32_t param_dtype;
  int64_t grad_base;
  void* param;               /* device working copy; param[j - param_base] for j in [s_k, e_k) */
  int64_t param_base;
  void* g16_dev;             /* device, L_k elements: the rounded mean before it is copied */
  float* partial;            /* device fp32, L_k elements: needed when p > ZS_KERNARG_P */
  /* host side (pinned memory, e.g. hipHostMalloc, lets the copies overlap) */
  void* g16_host[2];         /* L_k elements each: gradients received (two slots) */
  float* w;                  /* fp32 master weights, L_k */
  float* m;                  /* moments as the form needs them (see zs_adam_form) */
  float* v;
  void* param_host;          /* L_k elements of param_dtype: updated parameters, staged */
  int64_t bucket_elems;      /* elements per bucket; 0: the whole shard is one bucket */
  int32_t threads;           /* CPU threads for the update (as zs_cpu_adam_step) */
  int32_t reserved;          /* must be 0 */
  void* compute_stream;      /* hipStream_t of the GPU mean */
  void* d2h_stream;          /* hipStream_t of the gradient copies */
  void* h2d_stream;          /* hipStream_t of the parameter copies */
} zs_offload_args;

/* One step of the offloaded update of rank k's shard, in `mode`, receiving
 * into g16_host[slot] (slot 0 or 1).  Per bucket: the rank-order fp32 mean
 * rounded to grad_dtype (zs_reduce_scatter_mean_local16) on compute_stream;
 * its copy to the host on d2h_stream once the mean is done; the update of the
 * bucket on the calling thread (zs_cpu_adam_step, bit for bit the GPU step's
 * arithmetic on the widened 16-bit gradient); the bucket's parameters to the
 * device on h2d_stream.  Returns when all of it is complete.  The working
 * copy outside [s_k, e_k) is not touched; in ZS_OFFLOAD_RECEIVE nothing but
 * g16_dev and g16_host[slot] is written.
 * Errors: ZS_ERR_NULL, ZS_ERR_ARG (mode, slot, p, k, n, hparams, more than
 * 4096 buckets), ZS_ERR_DTYPE, ZS_ERR_RANGE, ZS_ERR_ALIAS (device outputs
 * overlapping each other or a gradient range; host buffers overlapping each
 * other), ZS_ERR_UNSUPPORTED (no AVX2/F16C), ZS_ERR_HIP. */
zs_status zs_offload_step(const zs_offload_args* args, const zs_adam_hparams* hp, int32_t mode,
                          int32_t slot);

#ifdef __cplusplus
}
#endif

#endif /* ZSHARD_H */
