/*
 * cdrge.h - C ABI of the MI355X (gfx950) CD-RGE hot path.
 *
 * One CD-RGE update step, as described for arXiv 2505.17852 ("Scaling Recurrent Neural Networks
 * to a Billion Parameters with Zero-Order Optimization"):
 *
 *   losses:  L(theta + eps p_i), L(theta - eps p_i) for K Rademacher probes p_i, each the mean
 *            next-token cross-entropy of a full LSTM forward pass (pith.science review, "What
 *            carries the argument": only scalar losses return; alex-wiki source note, "Method":
 *            complete recurrent forwards at perturbed weights, no differentiation through time);
 *   update:  theta <- theta - eta / (2 K eps) * sum_i (L(theta + eps p_i) - L(theta - eps p_i)) p_i
 *            (the review's update is the eta = eps case of the alex-wiki g-hat form), with every
 *            p_i regenerated from its seed (alex-wiki "Method": reconstructible random seeds).
 *
 * The split between cdrge_probe_losses and cdrge_update follows the pages' distributed scheme
 * (review, "What carries the argument": workers compute perturbed losses and return only scalar
 * losses; the update needs only those scalars and the seeds).
 *
 * Model (the pages say only "LSTM", next-character prediction): embedding Emb[V][E] -> n_layers
 * LSTM layers (gate rows i, f, g, o; one bias per layer; zero initial state) -> W_out[V][H] +
 * b_out[V] -> softmax cross-entropy of token t+1 given tokens 0..t. Loss = mean over B*T.
 * Flat parameter layout, tensor ids in order: 0 Emb[V][E]; per layer l: 1+3l W_ih[4H][in_l]
 * (in_0 = E, in_l = H), 2+3l W_hh[4H][H], 3+3l b[4H]; 1+3L W_out[V][H]; 2+3L b_out[V];
 * row-major, concatenated.
 *
 * Probe signs: seed_i = Philox4x32-10(key = base_seed, counter = (i, lo32(step), hi32(step), 1)),
 * words 0 | 1 << 32. Element (tensor t, row r, column c) of p_i: word (c >> 5) & 3, bit
 * ((c & 31) >> 1) | ((c & 1) << 4) of Philox4x32-10(key = seed_i, counter = (c >> 7, r, t, 0));
 * a set bit is -1, a clear bit +1.
 *
 * Precision. dtype F32: parameters, arithmetic and losses in float32. dtype BF16: parameters
 * stored as bf16; a perturbed weight is bf16(float(w) +- eps) rounded to nearest even; matrix
 * products take bf16 operands (activations are rounded to bf16 where they enter a product) and
 * accumulate in float32; cell state, gates, logits and losses are float32; the update adds in
 * float32 and rounds to bf16. dtype BF16_EXACT: as BF16, but the probe is added exactly (below).
 *
 * Conventions shared by every call:
 *   - Pointers named as device pointers must be device memory of the GPU that was current at
 *     cdrge_init; the caller owns them (the library never allocates or frees device memory).
 *   - Work is enqueued on the stream given to cdrge_init (a hipStream_t passed as void*; NULL is
 *     the default stream) and calls return after enqueueing. Only cdrge_sync_status waits.
 *   - Argument errors are reported synchronously and enqueue nothing. A failed launch returns
 *     CDRGE_ERR_DEVICE. A context is bound to one stream and is not thread-safe.
 */
#ifndef CDRGE_H
#define CDRGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CDRGE_ABI_VERSION 1u

typedef struct cdrge_ctx cdrge_ctx; /* opaque, host memory, owned by the library */

typedef enum {
  CDRGE_OK = 0,
  CDRGE_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, wrong abi_version, ... */
  CDRGE_ERR_UNSUPPORTED = 2, /* valid configuration that the kernels do not tile */
  CDRGE_ERR_WORKSPACE = 3,   /* workspace missing, too small or misaligned */
  CDRGE_ERR_DEVICE = 4,      /* a HIP runtime call or kernel launch failed */
  CDRGE_ERR_NONFINITE = 5    /* a probe loss was NaN or infinite; the update left theta as is */
} cdrge_status;

/* CDRGE_BF16_EXACT: bf16 parameters with the probe added exactly. A radius eps below the bf16
 * spacing of a weight (eps = 1e-4 against |w| around 2^-6 .. 2^-5) is swallowed when the perturbed
 * weight is rounded back to bf16; here every matrix product takes the stored weights W and the
 * exact bf16 operand eps' P, eps' = bf16(eps), into the same float32 accumulator:
 * (W +- eps' P) x = W x +- eps' (P x), twice the matrix-core work of CDRGE_BF16. Biases get
 * +- eps' p in float32; the perturbed embedding rows are rounded to bf16 (they are the first
 * product's activations); activations are rounded as for CDRGE_BF16. The update uses
 * eta / (2 K eps'), the radius actually applied. (alex-wiki source note, "Method": weights
 * perturbed by eps u_i; the pages fix no precision.) */
typedef enum { CDRGE_F32 = 0, CDRGE_BF16 = 1, CDRGE_BF16_EXACT = 2 } cdrge_dtype;

typedef struct {
  uint32_t abi_version;     /* must be CDRGE_ABI_VERSION */
  int32_t n_layers;         /* L >= 1 */
  int32_t vocab;            /* V */
  int32_t embed;            /* E */
  int32_t hidden;           /* H */
  int32_t batch;            /* B sequences per forward */
  int32_t seq_len;          /* T predicted positions; tokens are [B][T+1] */
  int32_t n_probes;         /* K probe pairs: 2K forwards per step */
  int32_t probes_per_chunk; /* probe pairs evaluated together; 0 = all K. Results do not depend on it */
  int32_t dtype;            /* cdrge_dtype */
  float eps;                /* probe radius */
  float lr;                 /* eta; the pages' runs use eta = eps */
  uint64_t base_seed;       /* root of the probe seed stream */
} cdrge_config;

/* Number of parameters d in the flat layout above, or -1 for an invalid configuration. */
int64_t cdrge_param_count(const cdrge_config* cfg);

/* CDRGE_OK if the configuration is valid and supported; otherwise the reason.
 * Supported: n_probes <= 1024, and
 *   F32 with n_layers <= 8 and E, H, V <= 65536 when the on-chip state of one workgroup - h and c
 *   of every layer, the gate pre-activations, the layer input and its tables of signed partial
 *   sums for up to 2 probe pairs x 8 sequences - fits in 128 KB (about
 *   4 * m * (2 L H + 5 max(E, H) + 4 H) bytes for m = 2 * pairs * sequences per workgroup, plus
 *   8 L H bytes of biases);
 *   BF16 and BF16_EXACT when E % 32 == 0, H % 32 == 0, V <= 64, and one probe chunk's activations stay within
 *   32-bit element offsets: (2 * probes_per_chunk * B + 256) * max(E, H) < 2^31 and
 *   4 H max(E, H) < 2^31. */
cdrge_status cdrge_check_config(const cdrge_config* cfg);

/* Device workspace, in bytes, that cdrge_init needs for this configuration (256-byte aligned
 * base required). It holds the probe seeds, per-step perturbation tables and the recurrent state
 * of one probe chunk; its size grows with probes_per_chunk. */
cdrge_status cdrge_workspace_bytes(const cdrge_config* cfg, size_t* bytes_out);

/* The K probe seeds of update step `step`, computed on the host into seeds_host[K]. */
cdrge_status cdrge_probe_seeds(const cdrge_config* cfg, uint64_t step, uint64_t* seeds_host);

/* Creates a context. params: device pointer to the d parameters (float32 or bf16 bit patterns,
 * per dtype), updated in place by cdrge_update. workspace: device pointer of at least
 * cdrge_workspace_bytes. stream: hipStream_t. Both buffers must outlive the context. */
cdrge_status cdrge_init(cdrge_ctx** ctx_out, const cdrge_config* cfg, void* params,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Enqueues the 2K perturbed forward passes of step `step`.
 *   tokens: device int32 [B][T+1]; every entry must lie in [0, V) (checked on the device:
 *     an out-of-range token makes the step's losses NaN).
 *   losses: device float32 [2K]; losses[2i] = L(theta + eps p_i), losses[2i+1] = L(theta - eps p_i).
 *   seq_losses: device float32 [2K][B] or NULL; per-sequence sums over t of the cross-entropy.
 * theta is read only. */
cdrge_status cdrge_probe_losses(cdrge_ctx* ctx, const int32_t* tokens, uint64_t step,
                                float* losses, float* seq_losses);

/* Enqueues the update of step `step` from device losses[2K] (layout as above). If any loss is
 * not finite, theta is left unchanged and the next cdrge_sync_status reports
 * CDRGE_ERR_NONFINITE. */
cdrge_status cdrge_update(cdrge_ctx* ctx, uint64_t step, const float* losses);

/* cdrge_probe_losses followed by cdrge_update on the same stream. */
cdrge_status cdrge_step(cdrge_ctx* ctx, const int32_t* tokens, uint64_t step, float* losses);

/* Transduction form of cdrge_probe_losses, for the synthetic sequence-to-sequence tasks the pages
 * also train on (alex-wiki source note, "Evidence And Limits": copy, reverse and rolling sum,
 * where only the output part of a sequence is scored).
 *   inputs: device int32 [B][T], every entry in [0, V): the token fed at (b, t).
 *   targets: device int32 [B][T]: the token to predict at (b, t), in [0, V), or below zero for a
 *     position that is not scored.
 * The loss of a perturbed model is the mean cross-entropy over the scored positions of the batch
 * (NaN when none is scored or an entry is out of range); seq_losses, when not NULL, gets the
 * per-sequence sums over the scored positions. cdrge_probe_losses(tokens) is this call with
 * inputs = tokens[:, 0:T] and targets = tokens[:, 1:T+1]. */
cdrge_status cdrge_probe_losses_io(cdrge_ctx* ctx, const int32_t* inputs, const int32_t* targets,
                                   uint64_t step, float* losses, float* seq_losses);

/* cdrge_probe_losses_io followed by cdrge_update on the same stream. */
cdrge_status cdrge_step_io(cdrge_ctx* ctx, const int32_t* inputs, const int32_t* targets, uint64_t step,
                           float* losses);

/* Waits for the context's stream and reports deferred errors (non-finite losses, device
 * faults). Clears the non-finite flag. */
cdrge_status cdrge_sync_status(cdrge_ctx* ctx);

/* Releases the context (host memory only). */
void cdrge_destroy(cdrge_ctx* ctx);

/* Static, human-readable name of a status. */
const char* cdrge_status_string(cdrge_status status);

/* Text of the last HIP failure behind a CDRGE_ERR_DEVICE returned to the calling thread
 * ("" if none). The pointer stays valid until the thread's next failing call. */
const char* cdrge_last_error_detail(void);

/* Diagnostics: when enabled, every launch is bracketed by HIP events on the context's stream
 * and its duration is added to a per-kind total. kind: 0 recurrent gate kernel, 1 logits and
 * cross-entropy, 2 update, 3 per-step preparation and loss reduction. The events are timing-only
 * (created without a system-scope fence), so recording them adds no cache write-back between
 * kernels; they order nothing for other streams or the host. */
cdrge_status cdrge_set_timing(cdrge_ctx* ctx, int enable);

/* Total milliseconds and launch count per kind since the last reset (waits for the stream). */
cdrge_status cdrge_get_timing(cdrge_ctx* ctx, int kind, double* total_ms, int64_t* launches,
                              int reset);

/* Algorithmic work of the launches counted under `kind` so far: matrix-core flops for kinds 0
 * and 1 (2 * M * N * K of each product actually executed), bytes of parameters read and written
 * for kind 2. */
cdrge_status cdrge_get_work(cdrge_ctx* ctx, int kind, double* work);

/* Name of the kernel whose launches are timed under `kind` for this context's configuration
 * (kind 0: k_lstm_gates_bf16, k_lstm_f32 or k_lstm_f32_sliced; 1: k_logits_ce_bf16,
 * k_ce_f32_sliced, or "" when the persistent fp32 kernel computes the loss itself; 2: the update
 * kernel; 3 and invalid arguments: ""). Static storage, never freed. */
const char* cdrge_timed_kernel(const cdrge_ctx* ctx, int kind);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): one whole step, as cdrge_step, with no context and no
 * caller workspace. The workspace lives in a static device array of the library, one per device
 * (held from library load until the process ends), of cdrge_noalloc_max_workspace_bytes()
 * bytes (64 MiB): configurations whose cdrge_workspace_bytes exceed it are rejected with
 * CDRGE_ERR_WORKSPACE before anything is enqueued (smaller probes_per_chunk shrinks the need).
 * The call allocates nothing: no hipMalloc, no hipFree, no library allocation of device memory.
 * params, tokens and losses are as for cdrge_init, cdrge_probe_losses and cdrge_step; stream is a
 * hipStream_t (NULL: the default stream). Every call on one device shares that device's array and
 * finds it as the previous call left it (the status words are cleared at the start of each call),
 * so calls that overlap on one device - on two streams, or from two threads - race and must be
 * ordered by the caller. A non-finite loss leaves theta unchanged; with no context, the caller
 * reads that from the losses it gets back. */
cdrge_status cdrge_step_noalloc(const cdrge_config* cfg, void* params, const int32_t* tokens,
                                uint64_t step, float* losses, void* stream);

/* Size in bytes of the static per-device scratch cdrge_step_noalloc uses. */
size_t cdrge_noalloc_max_workspace_bytes(void);

#ifdef __cplusplus
}
#endif

#endif /* CDRGE_H */
