/*
 * muon.h -- C ABI of the MI355X (gfx950) Muon optimizer step.
 *
 * One call runs the whole Muon step over a list of 2-D weight matrices:
 *   M' = beta*M + G                        (momentum, no dampening)
 *   U  = M'   (or beta*M' + G with MUON_FLAG_NESTEROV)
 *   X0 = U / (||U||_F + eps)               (Frobenius normalization)
 *   X  <- a_k X + (b_k A + c_k A A) X,  A = X X^T,  k = 1..ns_steps
 *         (on the smaller side: matrices with rows > cols are transposed)
 *   W' = (1 - lr*wd) W - lr * s_rule(rows, cols) * X
 * It also runs the AdamW step for the other parameters (muon_adamw_step) and
 * the Muon-Cayley step on the Stiefel manifold (muon_cayley_step).
 * Sources, cited by page title and section:
 *   [Muon优化器] linsight.cn/f25d614e.html -- the industrial Muon class
 *     (momentum, Nesterov, decay and apply), zeropower_via_newtonschulz
 *     (normalization, transposition, the quintic iteration) and section
 *     "缩放因子：从初始化到更新尺度" (the four scale rules);
 *   [DeepSeek V4 summary] prism.simon-ai.net/article/8795, section
 *     "Muon的训练效率与DeepSeek V4的混合优化策略" -- per-step coefficients
 *     (8 fast iterations, then 2 stable ones);
 *   [Adam vs Muon essay] guanweilu.cn/article/354.html -- the step as
 *     muon_step(weight, grad, momentum, lr, beta).
 *
 * Conventions for every entry point:
 *  - Matrices are dense, row-major, contiguous, rows = d_out, cols = d_in
 *    (the PyTorch Linear layout), in device memory of the current HIP
 *    device.  All matrices of one call share one dtype (hp->dtype).
 *  - The caller owns every device buffer, including the workspace; the
 *    library never allocates device memory in these calls and keeps no
 *    pointer once the enqueued work has finished.  Host arrays (mats,
 *    hp->schedule) are read during the call only.
 *  - `stream` is a hipStream_t passed as void*; NULL means the default
 *    stream.  Work is enqueued asynchronously; device buffers must stay
 *    alive until the stream reaches that point.
 *  - Argument validation is synchronous and happens before anything is
 *    enqueued; on any error nothing is modified.  Faults during kernel
 *    execution surface at the caller's next synchronization.
 *  - NaN/Inf in G or M are not checked; they stay inside their own matrix.
 *  - Not re-entrant on one workspace: concurrent calls need separate
 *    workspaces (and, if they must overlap, separate streams).
 */
#ifndef MUON_MI355X_H
#define MUON_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MUON_OK = 0,
    MUON_ERR_INVALID_ARG = -1,  /* bad pointer, shape, enum, non-finite scalar, overlap */
    MUON_ERR_UNSUPPORTED = -2,  /* device is not gfx950, or a size beyond the limits below */
    MUON_ERR_WORKSPACE = -3,    /* workspace NULL, too small or not 256-byte aligned */
    MUON_ERR_HIP = -4           /* a HIP runtime call or kernel launch failed */
} muon_status;

typedef enum { MUON_F32 = 0, MUON_BF16 = 1 } muon_dtype;

/* [Muon优化器] section "缩放因子：从初始化到更新尺度" (d_out = rows, d_in = cols):
 *   NAIVE         1
 *   KELLER_JORDAN sqrt(max(1, d_out/d_in))
 *   MUP           sqrt(d_out/d_in)
 *   MOONLIGHT     0.2 * sqrt(max(d_out, d_in))                               */
typedef enum {
    MUON_SCALE_NAIVE = 0,
    MUON_SCALE_KELLER_JORDAN = 1,
    MUON_SCALE_MUP = 2,
    MUON_SCALE_MOONLIGHT = 3
} muon_scale_rule;

/* One Newton-Schulz step's coefficients: X <- a X + (b A + c A A) X. */
typedef struct { float a, b, c; } muon_ns_coeffs;

/* Nesterov form: the iteration runs on beta*M' + G instead of M'
 * ([Muon优化器], industrial Muon class, nesterov branch). */
#define MUON_FLAG_NESTEROV 1u

/* Upper limits of this build. */
#define MUON_MAX_NS_STEPS 64
#define MUON_MAX_MATRICES 65536
#define MUON_MAX_DIM      (1 << 20)

typedef struct {
    void*       weight;    /* in/out, rows x cols */
    const void* grad;      /* in; NULL => the matrix is skipped entirely (state untouched) */
    void*       momentum;  /* in/out optimizer state, same dtype and shape */
    int64_t     rows, cols;
} muon_matrix;

typedef struct {
    float lr;                         /* finite */
    float beta;                       /* finite */
    float weight_decay;               /* finite */
    float eps;                        /* finite, >= 0; added to the Frobenius norm */
    int32_t scale_rule;               /* muon_scale_rule */
    int32_t ns_steps;                 /* 0..MUON_MAX_NS_STEPS; 0 => X = X0 */
    const muon_ns_coeffs* schedule;   /* host array of ns_steps triples (finite) */
    int32_t dtype;                    /* muon_dtype of weight, grad and momentum */
    uint32_t flags;                   /* MUON_FLAG_NESTEROV or 0 */
} muon_hparams;

/* Bytes of device workspace muon_step needs for this list (0 on invalid
 * arguments; the reason is in muon_last_error_message()).  Host-only. */
size_t muon_workspace_bytes(const muon_matrix* mats, int32_t n, const muon_hparams* hp);

/* One Muon step over `n` matrices, grouped: one launch per phase covers all
 * of them.  `workspace` is device memory of at least muon_workspace_bytes()
 * bytes, 256-byte aligned; its contents need not be initialized.
 * Writes weight and momentum of every matrix whose grad is non-NULL. */
muon_status muon_step(const muon_matrix* mats, int32_t n, const muon_hparams* hp,
                      void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): muon_step
 * with its workspace in a library-owned device array of
 * MUON_NOALLOC_SCRATCH_BYTES bytes per GPU.  The array is part of the
 * library's device code; its address is looked up on the first call on each
 * device, and each GPU the library runs on holds it until the process ends.
 * The call allocates nothing, on the device or the host: the descriptors
 * travel as kernel arguments.
 *  - A list whose muon_workspace_bytes() exceeds MUON_NOALLOC_SCRATCH_BYTES is
 *    rejected with MUON_ERR_WORKSPACE before anything is enqueued (128 MiB
 *    holds, for example, any one 2048 x 8192 matrix in bf16).
 *  - Every call on one GPU uses that GPU's one array, which keeps the last
 *    call's contents (nothing in it has to start at zero).  Calls that overlap
 *    on one GPU, from other streams or threads, race: the caller serializes them.
 *  - Validation, results and errors are otherwise those of muon_step. */
#define MUON_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
muon_status muon_step_noalloc(const muon_matrix* mats, int32_t n, const muon_hparams* hp, void* stream);

/* Orthogonalization only (the zeropower_via_newtonschulz contract of
 * [Muon优化器]): out = NS(in / (||in||_F + eps)) with hp's schedule.
 * `in` has hp->dtype; `out` is fp32, same shape, row-major; in and out must
 * not overlap.  hp's lr, beta, weight_decay, scale_rule and flags are ignored. */
typedef struct {
    const void* in;
    float*      out;
    int64_t     rows, cols;
} muon_ns_matrix;

size_t muon_ns_workspace_bytes(const muon_ns_matrix* mats, int32_t n, const muon_hparams* hp);
muon_status muon_ns(const muon_ns_matrix* mats, int32_t n, const muon_hparams* hp,
                    void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * AdamW for the parameters Muon does not take (embeddings, heads, biases,
 * norms), as one grouped launch over a list of tensors:
 *   m' = beta1 m + (1 - beta1) g
 *   v' = beta2 v + (1 - beta2) g^2
 *   p' = (1 - lr wd) p - lr (m' / (1 - beta1^t)) / (sqrt(v' / (1 - beta2^t)) + eps)
 * Sources: [Muon优化器] section "AdamW的问题" (moments, bias corrections, the
 * step); [DeepSeek V4 summary] section "Adam优化器的机制与AdamW的改进" (decay
 * apart from the gradient update); [Muon在Stiefel流形上的精确闭式更新解析]
 * section 4.3 (decay first, moments start at zero, t counts calls).
 * Arithmetic is fp32; p' is rounded once (RNE) to the parameter dtype.
 * --------------------------------------------------------------------------- */
typedef struct {
    void*       param;       /* in/out, numel elements of hp->dtype, contiguous */
    const void* grad;        /* in, same dtype; NULL => the tensor is skipped (state untouched) */
    float*      exp_avg;     /* in/out first moment, numel fp32 (zero before the first step) */
    float*      exp_avg_sq;  /* in/out second moment, numel fp32 (zero before the first step) */
    int64_t     numel;       /* >= 1, <= MUON_MAX_ADAMW_NUMEL */
} muon_adamw_tensor;

#define MUON_MAX_ADAMW_TENSORS 65536
#define MUON_MAX_ADAMW_NUMEL   ((int64_t)1 << 40)

typedef struct {
    float lr;            /* finite */
    float beta1, beta2;  /* in [0, 1) */
    float eps;           /* finite, >= 0 */
    float weight_decay;  /* finite */
    int32_t step;        /* t >= 1: this call is the t-th step of these tensors */
    int32_t dtype;       /* muon_dtype of param and grad */
} muon_adamw_hparams;

/* Device workspace bytes muon_adamw_step needs (0 on invalid arguments). */
size_t muon_adamw_workspace_bytes(const muon_adamw_tensor* tensors, int32_t n, const muon_adamw_hparams* hp);
/* One AdamW step over `n` tensors; the same validation, workspace and stream
 * rules as muon_step.  Tensors must not overlap each other or the workspace. */
muon_status muon_adamw_step(const muon_adamw_tensor* tensors, int32_t n, const muon_adamw_hparams* hp,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Muon-Cayley: the closed-form update that keeps a weight on the Stiefel
 * manifold ([Muon在Stiefel流形上的精确闭式更新解析], sections 1.3, 3.1-3.3, 6.2).
 * For W with orthonormal columns (W^T W = I; for rows < cols, orthonormal rows,
 * handled as the transpose):
 *   M' = beta M + (1 - beta) (G - 1 mean(G)^T)      mean over the rows
 *   V  = M' - W sym(W^T M'),   sym(S) = (S + S^T) / 2
 *   W' = (I + c A)^-1 (I - c A) W,  A = V W^T - W V^T,  c = lr / 2
 * computed through a 2k x 2k linear system (A has rank at most 2k,
 * k = min(rows, cols)).  fp32 buffers; the 2k x 2k solve runs in fp64.  For
 * k <= 128 it eliminates by k x k blocks and inverts the two diagonal blocks
 * by Gauss-Jordan without pivoting (on the manifold the symmetric part of each
 * is positive definite), switching to partial pivoting for a block whose
 * pivot falls below 1/2; for k > 128 it is an LU factorization with partial
 * pivoting.  No weight decay on this path.
 * --------------------------------------------------------------------------- */
typedef struct {
    float*       weight;    /* in/out rows x cols, fp32, row-major */
    const float* grad;      /* in; NULL => the matrix is skipped */
    float*       momentum;  /* in/out, same shape (zero before the first step) */
    int64_t      rows, cols;
} muon_cayley_matrix;

#define MUON_CAYLEY_MAX_K 256   /* min(rows, cols) limit of this build */

typedef struct {
    float lr;      /* finite */
    float beta;    /* in [0, 1) */
} muon_cayley_hparams;

size_t muon_cayley_workspace_bytes(const muon_cayley_matrix* mats, int32_t n, const muon_cayley_hparams* hp);
/* One Muon-Cayley step over `n` matrices (grouped launches).  Same workspace,
 * stream and validation rules as muon_step; min(rows, cols) above
 * MUON_CAYLEY_MAX_K is MUON_ERR_UNSUPPORTED. */
muon_status muon_cayley_step(const muon_cayley_matrix* mats, int32_t n, const muon_cayley_hparams* hp,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Static description of a status code. */
const char* muon_status_string(int32_t status);
/* Detail of the calling thread's last failure ("" if none). */
const char* muon_last_error_message(void);

/* Optional per-kernel timing with HIP events recorded on the launch stream.
 * While enabled, every launch of muon_step / muon_ns is bracketed by two
 * events; muon_profile_read synchronizes them and returns, per kernel class,
 * the summed duration in milliseconds and the number of launches, then
 * resets the counters.  Classes: 0 momentum+norm, 1 norm finalize, 2 Gram,
 * 3 polynomial, 4 update, 5 apply, 6 AdamW, 7 Muon-Cayley (all its kernels),
 * 8 the last update of muon_step, which also applies decay and the step to W.
 * Host-side bookkeeping only. */
#define MUON_KCLASS_COUNT 9
typedef struct {
    double  ms[MUON_KCLASS_COUNT];
    int64_t launches[MUON_KCLASS_COUNT];
} muon_profile;

muon_status muon_profile_enable(int32_t on);
muon_status muon_profile_read(muon_profile* out);

/* Library version as major*10000 + minor*100 + patch. */
int32_t muon_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MUON_MI355X_H */
