/*
 * zo.h -- C ABI of the multi-probe SPSA (zeroth-order) training step on one
 * AMD MI355X (gfx950).
 *
 * The step, as the pages state it (ZOO blog "Backprop 없이 Transformer를
 * 학습시킨다", section "backprop의 메모리 세금", loop flowchart, and section
 * "zero-order optimization이란"):
 *   for each of N random directions z_i: evaluate the loss at W + eps z_i and
 *   at W - eps z_i (forward only, no backprop); g_i = (L+_i - L-_i) / (2 eps);
 *   W <- W - eta * g_hat with g_hat = (1/N) sum_i g_i z_i; repeat.
 * Directions are Gaussian and rebuilt from a seed, never stored
 * ("0 차 최적화는 미탐구된 것이지, 저전력이 아니다", P1 and P5; FedSPZO
 * summary, section 2, "통신 프로토콜").  Training is in place, inference-mode:
 * the weights are the only model state (ZOO blog, 1.5-SPSA section).
 *
 * Direction stream: element j of direction i under step seed s is word j % 4
 * of Philox4x32-10(counter = (q lo, q hi, i, 0), key = (s lo, s hi)),
 * q = j / 4, mapped to a Gaussian by Box-Muller on word pairs (0,1) and (2,3):
 * u_r = ((x_even >> 8) + 1) 2^-24, u_t = (x_odd >> 8) 2^-24,
 * z_even = sqrt(-2 ln u_r) cos(2 pi u_t), z_odd = sqrt(-2 ln u_r) sin(2 pi u_t).
 *
 * Conventions for every entry point:
 *  - Pointers marked "device" are device memory the caller allocated and owns
 *    (e.g. from PyTorch); the library only borrows them for the call and never
 *    frees them.  "host" pointers are read before the call returns.
 *  - Work is enqueued on the caller's stream `s` (a hipStream_t; NULL is the
 *    default stream) and is asynchronous: results are valid after the caller
 *    synchronises that stream.  The library allocates no device memory.
 *  - Arguments are validated before anything is launched: an error return
 *    means nothing was enqueued (except ZO_ERR_HIP, which reports a failed
 *    launch).  No C++ exception crosses this boundary.  zo_last_error() gives
 *    a message for the last failure on the calling thread.
 *  - Storage rounding D: identity for fp32 weights, round to nearest even for
 *    bf16 weights.
 */
#ifndef ZO_H
#define ZO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* zo_stream; /* a hipStream_t */

typedef enum {
    ZO_OK = 0,
    ZO_ERR_INVALID = -1,     /* bad argument: null, size, alignment, overlap */
    ZO_ERR_UNSUPPORTED = -2, /* dtype or shape the library does not handle */
    ZO_ERR_HIP = -3,         /* a HIP launch or runtime call failed */
    ZO_ERR_NONFINITE = -4,   /* a loss was NaN or infinite */
    ZO_ERR_WORKSPACE = -5    /* workspace smaller than zo_workspace_bytes() */
} zo_status;

typedef enum { ZO_F32 = 0, ZO_BF16 = 1 } zo_dtype;

typedef enum { ZO_MODEL_LSQ = 0, ZO_MODEL_MLP = 1, ZO_MODEL_DECODER = 2 } zo_model_kind;

typedef enum { ZO_ACT_GELU = 0, ZO_ACT_RELU = 1 } zo_act;

typedef enum { ZO_MODE_INPLACE = 0, ZO_MODE_FUSED = 1, ZO_MODE_COPIES = 2 } zo_mode;

/*
 * Direction distribution of a model (zo_model_desc.dirs).
 *  ZO_DIRS_GAUSS: the Gaussian stream above.
 *  ZO_DIRS_Q8: 8-bit packed directions (the ZOO blog's 1.5-SPSA section names
 *    an 8-bit packing random generator with a fused unpack/apply kernel for
 *    OPT-30B in place; it gives no format).  Element j of direction i is byte
 *    j % 4 (least significant first) of word (j / 4) % 4 of
 *    Philox4x32-10(counter = (q lo, q hi, i, 1), key = (s lo, s hi)), q = j / 16,
 *    used as a code k into T[k] = Phi^-1((k + 1/2) / 256) / r, r^2 the mean of
 *    the 256 squared quantiles, rounded once to fp32: a 256-level quantised
 *    Gaussian with mean 0 and variance 1.  Perturb, update, replay and in-place
 *    steps support it for every model; copies steps and the evaluations that
 *    apply directions as the weights are read (zo_forward_loss with
 *    perturbations, fused steps) support it for decoders and return
 *    ZO_ERR_UNSUPPORTED for it on the fp32 models.
 */
typedef enum { ZO_DIRS_GAUSS = 0, ZO_DIRS_Q8 = 1 } zo_dirs;

/*
 * Model description.  Fields a kind does not use must be 0.
 *  LSQ:     loss = ||X W - Y||_F^2 / (2 batch); W [d_in][d_out] fp32.
 *  MLP:     loss = mean_b CE(GELU(X W1^T) W2^T, label_b); W1 [hidden][d_in],
 *           W2 [classes][hidden] fp32; no biases.
 *  DECODER: pre-LN decoder, bf16 weights: token embedding [vocab][d_model],
 *           learned positions [max_seq][d_model], per layer ln1 gain/bias [d],
 *           W_qkv [3d][d], W_o [d][d], ln2 gain/bias [d], W_up [ffn][d],
 *           W_down [d][ffn]; final LN gain/bias; LM head tied to the token
 *           embedding; no linear biases; act GELU (erf) or ReLU; loss = mean
 *           next-token CE over batch*(seq-1) positions.
 * `batch` (and `seq` for the decoder) is the largest batch forward_loss/step
 * will be given; it sizes the workspace.
 */
typedef struct {
    int32_t kind;  /* zo_model_kind */
    int32_t dtype; /* zo_dtype: F32 for LSQ/MLP, BF16 for DECODER */
    int64_t batch;
    int64_t seq;
    int64_t d_in, d_out;             /* LSQ, MLP (d_in) */
    int64_t hidden, classes;         /* MLP */
    int64_t layers, d_model, heads, ffn, vocab, max_seq; /* DECODER */
    int32_t act;                     /* zo_act, DECODER */
    int32_t dirs;                    /* zo_dirs: the direction distribution */
} zo_model_desc;

/* One parameter tensor inside the flat parameter arena. */
typedef struct {
    char name[32];
    uint64_t offset; /* element offset in the arena = its direction index */
    int64_t shape[2];
    int32_t ndim;
    int32_t reserved;
} zo_param_info;

/*
 * Batch.  Device pointers, row-major.
 *  LSQ: x fp32 [batch][d_in], y fp32 [batch][d_out].
 *  MLP: x fp32 [batch][d_in], labels int32 [batch] in [0, classes).
 *  DECODER: tokens int32 [batch][seq] in [0, vocab), seq <= max_seq.
 * `batch` and `seq` may be smaller than the model's maximum.
 */
typedef struct {
    const void* x;
    const void* y;
    const int32_t* labels;
    const int32_t* tokens;
    int64_t batch;
    int64_t seq;
} zo_batch;

/* A perturbation applied on the fly: weights seen = D(W + sigma * z_probe). */
typedef struct {
    uint64_t seed;
    uint32_t probe;
    float sigma;
} zo_pert;

typedef struct {
    uint64_t seed;     /* this step's direction seed */
    uint32_t n_probes; /* N >= 1 */
    float eps;         /* perturbation scale */
    float lr;          /* eta */
    int32_t mode;      /* zo_mode */
    int32_t precond;   /* 0: plain SPSA; 1: 1.5-SPSA (one clean evaluation per step) */
    float curv_floor;  /* 1.5-SPSA: lower bound of the curvature estimate, > 0 */
} zo_step_cfg;

/* Split-perturbation step configuration (zo_step_split). */
typedef struct {
    uint64_t seed; /* this step's direction seed */
    uint32_t p1;   /* theta_1 (W1) directions, >= 1 */
    uint32_t ps;   /* theta_2 (W2) directions per theta_1 branch, 1..4 */
    float eps;     /* perturbation scale of both blocks */
    float lr;      /* eta */
} zo_split_cfg;

/* Dust step configuration (zo_step_dust). */
typedef struct {
    uint64_t seed;  /* this step's noise seed */
    uint32_t k1;    /* hidden-layer draws, 1..128 */
    uint32_t k2;    /* head draws on the cached logits, 1..65536 */
    float sigma1;   /* hidden-layer noise scale */
    float sigma2;   /* logit noise scale */
    float lr;       /* eta */
} zo_dust_cfg;

typedef struct zo_model zo_model;

/* ---------------------------------------------------------------- layout */

/*
 * Parameter arena layout of a model: tensors in the order listed above, each
 * starting at a multiple of 64 elements; *total = arena length (a multiple of
 * 64).  Writes at most `cap` entries to `out` (host) and the count to *n_out.
 * Every arena element, padding included, is perturbed and updated; arena
 * element j uses direction element j.
 */
zo_status zo_param_layout(const zo_model_desc* desc, zo_param_info* out, int32_t cap, int32_t* n_out,
                          uint64_t* total);

/* Device workspace the model needs for its largest batch (bytes). */
zo_status zo_workspace_bytes(const zo_model_desc* desc, size_t* bytes);

/*
 * Creates a model over caller-owned device memory: `params` is the arena
 * (n_params elements of desc->dtype, 256-byte aligned, exactly the layout's
 * total), `workspace` at least zo_workspace_bytes() bytes (256-byte aligned).
 * Neither may overlap the other.  *out is a host object holding only
 * descriptors; release it with zo_model_destroy.
 */
zo_status zo_model_create(const zo_model_desc* desc, void* params, uint64_t n_params, void* workspace,
                          size_t ws_bytes, zo_model** out);
zo_status zo_model_destroy(zo_model* m);

/* ------------------------------------------------------------- the step */

/*
 * In-place perturbation of every parameter: w <- D(fma(sigma, z_probe, w)).
 * The +eps / -2 eps / +eps sequence restores W to within rounding.
 */
zo_status zo_perturb(zo_model* m, uint64_t seed, uint32_t probe, float sigma, zo_stream s);

/*
 * Forward-only loss evaluations (no activations kept beyond the call).
 * perts == NULL or n_perts == 0: one loss at the stored weights -> loss_dev[0].
 * Otherwise loss_dev[k] = loss at D(W + perts[k].sigma z_{perts[k].probe});
 * the weights in memory are not modified (the perturbation is applied inside
 * the kernels, tile by tile).  loss_dev: device, fp64, >= max(1, n_perts).
 * perts: host array.  With 8-bit directions only decoders take perturbations
 * (ZO_ERR_UNSUPPORTED otherwise).
 */
zo_status zo_forward_loss(zo_model* m, const zo_batch* b, const zo_pert* perts, int32_t n_perts,
                          double* loss_dev, zo_stream s);

/*
 * Fused update: c_i = fp32(-lr * g_i / N) from g_dev[0..N) (device, fp64),
 * then w <- D(w + sum_{i<N} c_i z_i) for every parameter, every z_i
 * regenerated from `seed`.  When any g_i is not finite nothing is written.
 */
zo_status zo_update(zo_model* m, uint64_t seed, uint32_t n_probes, const double* g_dev, float lr,
                    zo_stream s);

/*
 * One SPSA step.  mode INPLACE: for i < N: perturb(+eps), L+, perturb(-2 eps),
 * L-, perturb(+eps).  mode FUSED: every evaluation sees D(W +- eps z_i) of the
 * unmodified W (one launch covers all 2N evaluations where the model allows;
 * with 8-bit directions decoders only).
 * mode COPIES (decoder, Gaussian or 8-bit directions): the same evaluation weights as
 * FUSED, D(W +- eps z_i), written out: one pass over W fills 2P copies of the
 * arena for P probes, then one forward evaluates all 2P copies side by side
 * (the rows of every copy in the same launches); P is chosen so a forward
 * covers about 131072 token rows (at most 16 probes, at most N), and P = 1
 * unless batch * seq is a multiple of 256.  The copies and their workspace
 * (2P (arena + zo_workspace_bytes) bytes) are allocated on the model's first
 * COPIES step and held until zo_model_destroy; ZO_ERR_WORKSPACE if the device
 * cannot hold them for P = 1.  Losses equal FUSED's up to the order of the
 * GEMM accumulations; W changes only in the update.
 * Then g_i = (L+_i - L-_i) / (2 eps) and zo_update.
 * losses_dev: device fp64 [2N] as (L+_0, L-_0, L+_1, ...); g_dev: device fp64
 * [N].  A non-finite loss leaves W unchanged by the update (in place: after
 * the restore passes); the caller sees it in losses_dev / g_dev.
 * precond = 1 (1.5-SPSA: "1.5-SPSA" in the ZOO blog, section "첫 번째 논문:
 * probe-space 사전조건화"): one more evaluation L0 at the stored weights, first,
 * into losses_dev[2N] (losses_dev then holds 2N + 1 values); the probe-space
 * curvature h_i = (L+_i + L-_i - 2 L0) / eps^2 and g_dev[i] =
 * g_i / max(h_i, curv_floor), which the update uses in place of g_i.
 */
zo_status zo_step(zo_model* m, const zo_batch* b, const zo_step_cfg* cfg, double* losses_dev,
                  double* g_dev, zo_stream s);

/*
 * zo_step for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * validation, kernels and results as zo_step on a model created from `desc`
 * and `params` (params: the arena, n_params elements of desc->dtype, 256-byte
 * aligned, exactly the layout's total; device, caller-owned), but no
 * zo_model, no caller workspace and no allocation of any kind: the model's
 * workspace is a static 64 MiB device array inside the library, one per GPU,
 * held until the process ends (its address is looked up once per device, on
 * the first call with that device current).  Models whose workspace
 * (zo_workspace_bytes) exceeds 64 MiB are refused with ZO_ERR_WORKSPACE
 * (e.g. the least-squares and MLP workloads fit; a 12 x 768 decoder at
 * 8 x 512 tokens does not).  Every call on one GPU uses the same array:
 * calls that overlap on one GPU (concurrent streams or threads) race and give
 * undefined results; serialise them.  Nothing in the array needs to start at
 * zero.  With zo_timing_enable on, the timing bookkeeping allocates host
 * memory; leave it off here.  mode COPIES needs device memory of its own and
 * is refused here (ZO_ERR_UNSUPPORTED).
 */
zo_status zo_step_noalloc(const zo_model_desc* desc, void* params, uint64_t n_params, const zo_batch* b,
                          const zo_step_cfg* cfg, double* losses_dev, double* g_dev, zo_stream s);

/*
 * One split-perturbation step with activation reuse (FedSPZO summary,
 * section 2 "방법론"), for the MLP with d_in % 32 == 0 and Gaussian
 * directions.  theta_1 = W1 (with the GELU), theta_2 = W2.  For each theta_1
 * direction i < p1 and sign s (v = 0 for +, 1 for -) the block-1 output
 * y = GELU(X (W1 + s eps z1_i)^T) is formed once and reused by ps theta_2
 * directions z2_m, m = (2 i + v) ps + k, each evaluated at +eps and -eps:
 * losses_dev[2m] = L(y, W2 + eps z2_m), losses_dev[2m + 1] = L(y, W2 - eps z2_m)
 * (device fp64, 4 p1 ps values).  g2_dev[m] = (losses[2m] - losses[2m+1]) /
 * (2 eps) (device fp64, p2 = 2 p1 ps values); g1_dev[i] = (mean of branch
 * (i, +)'s 2 ps losses - mean of branch (i, -)'s) / (2 eps) (device, p1).
 * Then W1 <- W1 - (lr / p1) sum_i g1_i z1_i with z1_i = direction i, and
 * W2 <- W2 - (lr / p2) sum_m g2_m z2_m with z2_m = direction p1 + m, each on
 * its own tensor's elements only; a non-finite loss skips both.  The
 * evaluations use the linearity of both layers in their perturbation (W1's
 * product with X formed once; logits at W2 +- eps z2 as A W2^T +- eps A z2^T),
 * so they differ from products with rounded perturbed weights only by that
 * rounding.  ZO_ERR_UNSUPPORTED for other models, 8-bit directions,
 * d_in % 32 != 0, or (1 + ps) * classes > 56.
 */
zo_status zo_step_split(zo_model* m, const zo_batch* b, const zo_split_cfg* cfg, double* losses_dev,
                        double* g1_dev, double* g2_dev, zo_stream s);

/*
 * One Dust step (activation perturbation with per-token rewards; Dust review
 * page "Dust: 역전파 없이 트랜스포머를 사전학습하다", sections "Dust의 해법:
 * 가상 개체군", "신용 할당(credit assignment): 보상에서 기울기까지" and
 * "간섭(interference) 줄이기"), for the MLP with d_in % 32 == 0 and
 * batch % 32 == 0.  Every sample t is a token.  The clean forward is cached
 * (Y = X W1^T, A = GELU(Y), Z = A W2^T).  Hidden layer: k1 draws of noise
 * a ~ N(0, I) on Y (Philox counter stream 2, direction index = draw, element
 * t * hidden + h), per-token losses l_i[t]; reward r = lbar[t] - l_i[t];
 * output error ghat_t = -(1/(k1 sigma1)) sum_i r a_i[t]; W1 <- W1 - lr
 * sum_t ghat_t x_t^T.  Head: k2 draws of noise b on the cached logits (stream 3,
 * element t * classes + c), the same rewards, ghat2_t; W2 <- W2 - lr sum_t
 * ghat2_t A_t^T.  Both estimates come from the same weights; a non-finite loss
 * skips both updates.  losses_dev (device fp64, (1 + k1 + k2) * batch): the
 * clean per-token losses, then the k1 hidden draws', then the k2 head draws',
 * each [draw][token].  The step uses the model's workspace, which
 * zo_workspace_bytes sizes for k1 up to 128 at the model's batch.
 */
zo_status zo_step_dust(zo_model* m, const zo_batch* b, const zo_dust_cfg* cfg, double* losses_dev, zo_stream s);

/*
 * Seed replay of one recorded step (position paper summary, P5, and FedSPZO,
 * "통신 프로토콜": a model is rebuilt from the shared seeds and the scalar
 * gradients alone, no weights exchanged).  Applies to W exactly the weight
 * changes zo_step made with this cfg, given the g_dev [N] (device fp64) that
 * step produced: in place, the 3N perturb / restore passes in the step's order,
 * then the update; fused, the update only.  No evaluation runs, so no batch is
 * needed.  Starting from the same weights, replaying a step's records gives its
 * weights bit for bit (every kernel involved is deterministic); a checkpoint is
 * the initial weights plus (cfg, g) per step.  precond and curv_floor are not
 * read: g_dev already holds the scalars the update used.
 */
zo_status zo_replay_step(zo_model* m, const zo_step_cfg* cfg, const double* g_dev, zo_stream s);

/* ------------------------------------------------- model-free buffer path */

/*
 * The perturb and update passes on a raw buffer w (device, n elements of
 * `dtype`, 16-byte aligned) whose element 0 is direction element j0, with
 * directions of kind `dirs` (zo_dirs; j0 % 4 == 0 for ZO_DIRS_GAUSS,
 * j0 % 16 == 0 for ZO_DIRS_Q8).  Same arithmetic as zo_perturb / zo_update.
 */
zo_status zo_perturb_buffer(void* w, int32_t dtype, int32_t dirs, uint64_t n, uint64_t j0, uint64_t seed,
                            uint32_t probe, float sigma, zo_stream s);
zo_status zo_update_buffer(void* w, int32_t dtype, int32_t dirs, uint64_t n, uint64_t j0, uint64_t seed,
                           uint32_t n_probes, const double* g_dev, float lr, zo_stream s);

/* g_dev[i] = (losses_dev[2i] - losses_dev[2i+1]) / (2 (double)eps), i < n. */
zo_status zo_gscalar(const double* losses_dev, uint32_t n, float eps, double* g_dev, zo_stream s);

/* ---------------------------------------------------------------- debug */

/*
 * Direction elements j0 .. j0+n-1 of `probe` under `seed`: raw Philox words
 * (words_dev, uint32) and/or Gaussians (z_dev, fp32); either may be NULL.
 */
zo_status zo_debug_rng(uint64_t seed, uint32_t probe, uint64_t j0, uint64_t n, uint32_t* words_dev,
                       float* z_dev, zo_stream s);

/* Box-Muller map alone: pairs_dev [n][2] words -> z_dev [n][2] (z_even, z_odd). */
zo_status zo_debug_box_muller(const uint32_t* pairs_dev, uint64_t n_pairs, float* z_dev, zo_stream s);

/*
 * Single decoder kernels, for testing them in isolation (bf16 buffers, device):
 *  zo_debug_gemm_bf16: C[M][N] = epi(A[M][K] W[N][K]^T), fp32 accumulation,
 *    epi 0: bf16 store, 1: GELU then bf16, 2: ReLU then bf16,
 *    3: residual C = bf16(C + bf16(product)); K % 64 == 0, N % 8 == 0,
 *    A, W and C each under 2 GiB, buffers 16-byte aligned
 *    (ZO_ERR_UNSUPPORTED / ZO_ERR_INVALID otherwise).
 *  zo_debug_attention: out[B*S][H*dh] = causal softmax(Q K^T / sqrt(dh)) V per
 *    (sequence, head) from qkv[B*S][3*H*dh] (Q, K, V blocks of H*dh columns,
 *    head h at columns h*dh); dh in {64, 128}; qkv and out 16-byte aligned
 *    (ZO_ERR_INVALID otherwise), qkv under 2 GiB (ZO_ERR_UNSUPPORTED).
 *  zo_debug_layernorm: x[r] = bf16((h[r] - mean) / sqrt(var + 1e-5) * g + b).
 * The causal attention follows the decoder's definition (scale 1/sqrt(dh),
 * keys at positions <= the query's).
 */
zo_status zo_debug_gemm_bf16(const void* A_dev, const void* W_dev, void* C_dev, int32_t M, int32_t N, int32_t K,
                             int32_t epi, zo_stream s);
zo_status zo_debug_attention(const void* qkv_dev, void* out_dev, int32_t B, int32_t S, int32_t H, int32_t dh,
                             zo_stream s);
zo_status zo_debug_layernorm(const void* h_dev, const void* g_dev, const void* b_dev, void* x_dev, int32_t rows,
                             int32_t d, zo_stream s);

/* ------------------------------------------------------------ timing */

/*
 * Kernel timing, a measurement aid.  While enabled, every kernel launch of the
 * library is bracketed by HIP events recorded on the launch's own stream and
 * grouped by family: "perturb", "update", "gemm_f32" (fp32 GEMMs that carry
 * directions), "gemm_f32_base" (fp32 work on the stored weights alone: input
 * splitting, the stored product, clean evaluations), "reduce", "gemm_bf16",
 * "attention", "layernorm", "embed", "lm_head", "debug".  The decoder's layer
 * GEMMs are the sub-families "gemm_bf16.qkv", "gemm_bf16.o", "gemm_bf16.up" and
 * "gemm_bf16.down" of "gemm_bf16": a family name covers its sub-families
 * ("<family>.<name>") in both calls below.  zo_timing_query returns the summed
 * elapsed milliseconds and the launch count of one family since the last
 * reset; it synchronises the recorded events, so call it after the stream
 * work is complete.  zo_timing_select restricts the bracketing to one family
 * (NULL: every family), so that timing one kernel adds no events around the
 * others.  Not thread-safe across concurrent callers.
 */
zo_status zo_timing_enable(int32_t on);
zo_status zo_timing_select(const char* family);
zo_status zo_timing_reset(void);
zo_status zo_timing_query(const char* family, double* total_ms, int64_t* launches);

const char* zo_status_str(zo_status st);
const char* zo_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ZO_H */
