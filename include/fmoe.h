/*
 * fmoe.h -- C ABI of libfmoe.so: one decode step of a Mixture-of-Experts FFN
 * layer with 4-bit or 2-bit affine-quantised expert weights, on one AMD
 * Instinct MI355X (gfx950).
 *
 * The operation is the one described on the Flash-MoE pages:
 *   [WAS]  "Was ist Flash-MoE? 397B-Parameter-KI-Modelle auf einem Laptop
 *          laufen lassen" (a2a-mcp.org, German; zh/hi/pt translations)
 *   [HADA] "Flash-MoE - Ein 397-Milliarden-Parameter-Modell auf einem
 *          Notebook ausfuehren" (news.hada.io)
 * Per token: a router picks k routed experts plus one shared expert
 * ([WAS] "Verstaendnis von Mixture-of-Experts"); each expert is a
 * dequantised matrix-vector gate/up, SwiGLU, down chain over affine weights
 * w = code * scale + bias ([WAS] "2. FMA-optimierte Dequantisierungs-Kernel",
 * "3. Handoptimierte Metal Compute-Shader"); the results are combined with the
 * routing weights and a sigmoid-gated shared expert, added to the residual and
 * RMS-normalised for the next layer ([WAS] section 3, "MoE-Kombination +
 * Residual + Sigmoid-Gating"; [HADA] "Deferred GPU Expert Compute").
 *
 * Conventions common to every call
 * --------------------------------
 * Pointers: every tensor pointer is a DEVICE pointer owned by the caller.
 *   Descriptor structs (fmoe_qmat, fmoe_expert, fmoe_layer, fmoe_qformat) are
 *   host memory, read only during the call.  The library allocates and frees
 *   nothing on these paths and keeps no pointer after returning.
 * Streams: `stream` is a hipStream_t (NULL = the default stream).  Each call
 *   only enqueues kernels on it; no call copies between host and device or
 *   synchronises, so every call may be captured into a HIP graph.  Outputs are
 *   valid once the caller has synchronised with the stream.
 * Workspace: calls that take `ws` need ws_bytes >= the matching *_workspace_size
 *   value.  The workspace must be zero-filled before its first use (for example
 *   allocated with torch.zeros); every call leaves the counters it uses at zero
 *   again, so a workspace can be reused for any later call of any shape that
 *   fits.  Two calls in flight at once must use different workspaces.
 * Errors: arguments are validated on the host before anything is enqueued.  An
 *   invalid argument returns its status, enqueues nothing and sets the
 *   thread-local message returned by fmoe_last_error().  A failed launch returns
 *   FMOE_ERR_HIP with HIP's error text.  Faults during kernel execution surface
 *   at the caller's next synchronisation.  The library never aborts and no C++
 *   exception crosses this interface.  NaN and Inf inputs are propagated, not
 *   checked.
 * Quantised matrices: W[n, k] is stored row-major by output row n with the
 *   input dim k contiguous.  Codes are unsigned (0..2^bits-1) and packed
 *   LSB-first: element k of a row sits in byte k*bits/8 at bit position
 *   (k mod (8/bits))*bits.  scale and bias are [n, k/group] arrays of fp32 or
 *   bf16 (the same dtype for both); dequantised w = code * scale + bias.
 *   Supported: bits in {2, 4}; group in {32, 64}; k a multiple of group with
 *   k*bits/8 a multiple of 16; with S = k*bits/128 (16-byte segments per row),
 *   either S divides 64 or S is 64, 128 or 256.  q, scale and bias must be
 *   16-byte aligned.
 * Arithmetic: dot products accumulate in fp32.  Activations enter the
 *   dequantised products as fp16 values with a power-of-two scale per block
 *   of 32 (no overflow for any finite input); router logits accumulate in
 *   fp64 so that expert selection is exact.  Calls with T > 1 run 4-bit
 *   experts on the matrix cores, which form each dequantised weight in fp16
 *   from fp16 copies of its scale and bias: the scales and biases of one weight
 *   row (the gate and up rows of one index together) are first multiplied by
 *   the power of two that puts the row's largest |scale| or |bias| in
 *   [2^10, 2^11), and the fp32 result by its inverse.  Any finite fp32/bf16
 *   scale or bias is therefore in range; a value more than 2^24 times smaller
 *   than the largest of its row is held as an fp16 subnormal (less precise).
 *   fmoe_paths.no_mfma keeps such batches on the GEMV kernels, which apply
 *   scales and biases in fp32.
 */
#ifndef FMOE_H
#define FMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FMOE_ABI_VERSION 1

typedef enum {
    FMOE_OK = 0,
    FMOE_ERR_NULL = 1,        /* a required pointer is NULL */
    FMOE_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
    FMOE_ERR_ALIGN = 3,       /* a pointer or stride is not aligned as required */
    FMOE_ERR_UNSUPPORTED = 4, /* a format or shape this build does not implement */
    FMOE_ERR_WORKSPACE = 5,   /* ws is NULL or smaller than required */
    FMOE_ERR_HIP = 6          /* a HIP launch failed */
} fmoe_status;

typedef enum { FMOE_F32 = 0, FMOE_BF16 = 1 } fmoe_dtype;

/* Quantisation format: bits in {2,4}; group in {32,64} along the input dim;
 * sdtype (fmoe_dtype) is the storage type of both scale and bias. */
typedef struct {
    int32_t bits;
    int32_t group;
    int32_t sdtype;
} fmoe_qformat;

/* One quantised matrix W[n, k] (see "Quantised matrices" above). */
typedef struct {
    const void *q;
    const void *scale;
    const void *bias;
    int32_t n;
    int32_t k;
} fmoe_qmat;

/* One expert: gate and up are [inter x hidden], down is [hidden x inter]. */
typedef struct {
    fmoe_qmat gate, up, down;
} fmoe_expert;

/* One MoE layer whose experts are stored as slabs.  An expert slab holds
 * gate.q gate.scale gate.bias up.q up.scale up.bias down.q down.scale down.bias
 * in this order, each section starting on a 256-byte boundary (offsets from
 * fmoe_slab_layout); [HADA] "SSD Expert Streaming" describes one expert as the
 * unit that is read (about 6.75 MB at hidden 4096 / inter 1024, 4-bit, which
 * this layout reproduces).  `slabs` holds n_experts + 1 slabs of slab_stride
 * bytes; slab n_experts is the shared expert. */
typedef struct {
    int32_t hidden;              /* H */
    int32_t inter;               /* I, expert intermediate size */
    int32_t n_experts;           /* E routed experts */
    int32_t top_k;               /* k routed experts per token, 1 <= k <= min(E, 16) */
    fmoe_qformat fmt;            /* format of every expert matrix */
    const float *router_w;       /* [E, H] fp32 router weights, row-major */
    const void *slabs;           /* (E+1) * slab_stride bytes, 256-byte aligned */
    int64_t slab_stride;         /* bytes, a multiple of 256, >= fmoe_slab_layout() */
    const float *shared_gate_w;  /* [H] fp32: shared-expert gate g = sigmoid(w . x) */
    const float *norm_w;         /* [H] fp32 RMSNorm weight gamma */
    float norm_eps;              /* RMSNorm epsilon (1e-6 in the configs here) */
} fmoe_layer;

/* Kernel-path selection, for cross-checking one path against another and for
 * debugging; normal use never changes it.  The library reads the initial
 * values once, when it is loaded, from the environment:
 *   FMOE_NO_FUSED=1         multi-launch forms instead of the one-launch layer
 *                           (T == 1) and single-expert kernels
 *   FMOE_NO_MFMA=1          every expert of a batch on the multi-token GEMV
 *                           kernels instead of the matrix cores
 *   FMOE_MFMA_MIN_TOKENS=n  only experts with at least n tokens of a batch on
 *                           the matrix cores, the rest on the GEMV kernels
 *                           (default 1: every expert of a 4-bit batch)
 *   FMOE_DEBUG_SYNC=1       every call synchronises its stream before returning
 *                           and reports a kernel fault as FMOE_ERR_HIP (not
 *                           usable under graph capture)
 * The setting is process-wide; change it only while no call is in progress.
 * fmoe_set_paths returns FMOE_ERR_SHAPE for mfma_min_tokens < 1 or a negative
 * wait_limit_us or test_stall_part. */
typedef struct {
    int32_t no_fused;
    int32_t no_mfma;
    int32_t mfma_min_tokens;
    int32_t debug_sync;
    int32_t t1_counters;     /* 1: the one-token layer on the arrival-counter kernel instead
                                of the self-checking-record kernel (FMOE_T1_COUNTERS=1) */
    int32_t wait_limit_us;   /* bound of one in-kernel wait in microseconds; 0 = 200000
                                (FMOE_WAIT_LIMIT_US) */
    int32_t test_stall_part; /* tests of the timeout path only: n > 0 makes down part n-1 of
                                the one-token kernel never publish, so the waits for it give
                                up (bounded) and the call's outputs are NaN; 0 = off */
} fmoe_paths;
void fmoe_get_paths(fmoe_paths *paths);
fmoe_status fmoe_set_paths(const fmoe_paths *paths);

/* Version of this interface (FMOE_ABI_VERSION). */
int32_t fmoe_abi_version(void);

/* Message for the last non-OK status returned on the calling thread. */
const char *fmoe_last_error(void);

/* Diagnostics: byte offset, within any workspace, of the 32-bit word that the
 * one-launch kernels set to 1 when one of their bounded waits for another
 * workgroup gives up instead of hanging (the call's outputs are then not
 * valid).  It stays 0 otherwise; the caller may read it and clear it. */
size_t fmoe_wait_timeout_offset(void);

/* Section offsets off[9] of an expert slab in the canonical layout and the
 * slab size in bytes (the return value; -1 with the message set if the
 * arguments are unsupported).  Host-only; enqueues nothing. */
int64_t fmoe_slab_layout(int32_t hidden, int32_t inter, const fmoe_qformat *fmt,
                         int64_t off[9]);

/* Router and top-k for T tokens ([WAS] "Verstaendnis von Mixture-of-Experts":
 * k routed experts chosen per token).  logits[t,e] = sum_h router_w[e,h] *
 * x[t,h], accumulated in fp64.  The k experts with the largest logits are
 * returned in idx[t, 0..k-1] ordered by (logit descending, index ascending),
 * so a tie goes to the lower index.  w[t,i] is the softmax over all E logits
 * renormalised over the selection (equal to the softmax over the k selected
 * logits) and sums to 1.  logits_out ([T,E] fp32) may be NULL.
 *   router_w [E,H] fp32, x [T,H] fp32, idx [T,k] int32, w [T,k] fp32.
 *   H a multiple of 4, all pointers 16-byte aligned, 1 <= k <= min(E, 16),
 *   E <= 2048, H <= 8192 (FMOE_ERR_UNSUPPORTED beyond).  T == 0 is a no-op.
 *   ws: fmoe_route_workspace_size(T, E) bytes. */
fmoe_status fmoe_route_topk(const float *router_w, const float *x, int32_t T, int32_t H,
                            int32_t E, int32_t k, int32_t *idx, float *w, float *logits_out,
                            void *ws, size_t ws_bytes, void *stream);
size_t fmoe_route_workspace_size(int32_t T, int32_t E);

/* y[n] = sum_k (code[n,k] * scale[n,k/G] + bias[n,k/G]) * x[k]  for one
 * quantised matrix ([WAS] "3. Handoptimierte Metal Compute-Shader": 4-bit /
 * 2-bit tiled matrix-vector multiply).  x [W->k] fp32, y [W->n] fp32, both
 * 16-byte aligned; y must not overlap x.  No workspace. */
fmoe_status fmoe_dequant_gemv(const fmoe_qmat *W, const fmoe_qformat *fmt, const float *x,
                              float *y, void *stream);

/* One expert FFN on one token: y = deq(down) (silu(deq(gate) x) * deq(up) x),
 * silu(z) = z / (1 + exp(-z)) ([WAS] section 3: fused SwiGLU).  gate/up must be
 * [I x H], down [H x I].  x [H], y [H] fp32, 16-byte aligned, not overlapping.
 *   ws: fmoe_expert_ffn_workspace_size(e, fmt) bytes. */
fmoe_status fmoe_expert_ffn(const fmoe_expert *e, const fmoe_qformat *fmt, const float *x,
                            float *y, void *ws, size_t ws_bytes, void *stream);
size_t fmoe_expert_ffn_workspace_size(const fmoe_expert *e, const fmoe_qformat *fmt);

/* The whole MoE layer for T tokens:
 *   route (as fmoe_route_topk) -> for each token, the k routed experts and the
 *   shared expert (slab E) run as in fmoe_expert_ffn ->
 *   moe[t]  = sum_i w[t,i] * FFN_{idx[t,i]}(x[t]) + g[t] * FFN_shared(x[t]),
 *             g[t] = sigmoid(shared_gate_w . x[t])
 *   h_out[t] = residual[t] + moe[t]                     (the new residual)
 *   y_out[t] = norm_w * h / sqrt(mean(h^2) + norm_eps)   (input of the next layer)
 * Indices never leave the device, so layers chain by passing y_out and h_out
 * of one call as x and residual of the next.
 *   x, residual, h_out, y_out: [T,H] fp32.  residual may alias x and h_out may
 *   alias residual; no other overlap.  idx_out [T,k] int32, w_out [T,k] fp32
 *   and moe_out [T,H] fp32 (before the residual) may each be NULL.
 *   ws: fmoe_workspace_size(L, T) bytes.  T == 0 is a no-op. */
fmoe_status fmoe_moe_layer_forward(const fmoe_layer *L, int32_t T, const float *x,
                                   const float *residual, float *h_out, float *y_out,
                                   int32_t *idx_out, float *w_out, float *moe_out,
                                   void *ws, size_t ws_bytes, void *stream);
size_t fmoe_workspace_size(const fmoe_layer *L, int32_t T);

/* T tokens through n_layers MoE layers in order ([HADA] "Deferred GPU Expert
 * Compute": each layer's combine, norm and residual feed the next layer on the
 * device).  Layer 0 takes x and residual; layer l > 0 takes y_out[l-1] as x and
 * h_out[l-1] as residual; each layer computes what fmoe_moe_layer_forward
 * computes, into row l of the outputs:
 *   x, residual [T,H] fp32 (residual may alias x); h_out, y_out [n_layers,T,H]
 *   fp32, overlapping neither x, residual nor each other; idx_out and w_out
 *   [n_layers,T,k] may each be NULL.  Every layer has the shape, format,
 *   slab_stride and norm_eps of layers[0] (FMOE_ERR_SHAPE otherwise); only the
 *   weight pointers differ.  ws: fmoe_workspace_size(&layers[0], T) bytes.
 *   n_layers == 0 or T == 0 is a no-op.
 * At T == 1 up to 64 layers run in one launch: the workgroups stay resident
 * from layer to layer and each builds the next layer's input in its own LDS
 * from the records of the last hand-off, so neither the launch gap nor a
 * round trip of x through memory separates two layers.  Other shapes run one
 * layer call after another; the results are the same. */
fmoe_status fmoe_moe_stack_forward(const fmoe_layer *layers, int32_t n_layers, int32_t T,
                                   const float *x, const float *residual, float *h_out,
                                   float *y_out, int32_t *idx_out, float *w_out, void *ws,
                                   size_t ws_bytes, void *stream);

/* One decode step of the Gated DeltaNet state update for `batch` sequences x
 * `heads` heads ([WAS] "4. Accelerate BLAS fuer Gated DeltaNet-Schichten": the
 * 64-head state matrix of a linear-attention layer updated by a scale, a
 * matrix-vector product and a rank-1 update).  Per (b, h), with the head's
 * state S [dk x dv] (row-major: S[i][j] at i*dv + j), key k and query q [dk],
 * value v [dv], decay a and write strength beta:
 *   S <- a S;   u = S^T k;   S <- S + beta k (v - u)^T;   out = S^T q.
 *   q, k [batch, heads, dk], v [batch, heads, dv], decay, beta [batch, heads],
 *   state [batch, heads, dk, dv] (updated in place), out [batch, heads, dv];
 *   all fp32; q, k, v, state and out 16-byte aligned.  dk in {32, 64, 128, 256},
 *   dv a positive multiple of 32 (FMOE_ERR_UNSUPPORTED otherwise).  out must
 *   not overlap anything, the state no input.  batch * heads == 0 is a no-op
 *   (no pointer is read or checked).
 * The step is one pass over the state (read once, written once), in fp32. */
fmoe_status fmoe_deltanet_step(const float *q, const float *k, const float *v,
                               const float *decay, const float *beta, float *state, float *out,
                               int32_t batch, int32_t heads, int32_t dk, int32_t dv, void *stream);

/* Decode attention of one new token per sequence over a bf16 KV cache, with
 * the query's rotary embedding applied on the fly ([WAS] "3. Handoptimierte
 * Metal Compute-Shader": GPU-side RoPE with the query de-interleaved, batched
 * attention for the full-attention layers; the products Q K^T, softmax and
 * scores V).  For sequence b, query head h and its KV head h / (n_q_heads /
 * n_kv_heads), with L = lens[b] cached positions (the new token's key and
 * value already at position L - 1) and D = head_dim:
 *   q'[i] = q[2i] cos t_i - q[2i+1] sin t_i,  q'[i + D/2] = q[2i] sin t_i + q[2i+1] cos t_i,
 *           t_i = (L - 1) rope_base^(-2i/D)
 *   out[b,h] = sum_t softmax_t(q' . K_t / sqrt(D)) V_t,   t < L.
 *   q [batch, n_q_heads, D] fp32 (rotation pairs interleaved, not yet rotated);
 *   k_cache, v_cache [batch, n_kv_heads, cap, D] bf16 bits (keys rotated, in
 *   half-split order); lens [batch] int32 DEVICE array with 1 <= lens[b] <= cap
 *   (read by the kernels: a length outside that range is clamped into [0, cap],
 *   and 0 gives NaN for that sequence); out [batch, n_q_heads, D] fp32.
 *   D in {64, 128, 256}; n_q_heads a multiple of n_kv_heads by at most 16.
 *   q, caches and out 16-byte aligned, out overlapping no input.
 *   ws: fmoe_attention_workspace_size(batch, n_kv_heads, D, cap) bytes,
 *   256-byte aligned, no initial contents needed.  batch == 0 is a no-op.
 * Q K^T runs on the matrix cores with the rotated query split into two bf16
 * halves (16 significant bits); the softmax and P V in fp32. */
fmoe_status fmoe_attention_decode(const float *q, const uint16_t *k_cache, const uint16_t *v_cache,
                                  const int32_t *lens, int32_t batch, int32_t n_q_heads,
                                  int32_t n_kv_heads, int32_t head_dim, int32_t cap,
                                  float rope_base, float *out, void *ws, size_t ws_bytes,
                                  void *stream);
size_t fmoe_attention_workspace_size(int32_t batch, int32_t n_kv_heads, int32_t head_dim,
                                     int32_t cap);

/* Host-tier expert streaming, for expert sets larger than HBM ([WAS] "1.
 * SSD-Experten-Streaming mit macOS Page Cache", [HADA] "SSD Expert Streaming":
 * only the experts a layer selects are read from the slower tier, and a cache
 * keeps recent ones).  The slower tier is pinned host memory; the faster one a
 * layer's slab array in HBM whose slot e holds expert e of whichever layer
 * last fetched it, recorded by the caller's tag in tags[e].  For every expert e
 * in idx[0 .. n_idx-1] and `shared` (a slot, or -1 for none), whose slot does
 * not already carry `tag`: copy host_slabs + e*slab_stride (slab_bytes bytes)
 * to dev_slabs + e*slab_stride; then tags[e] = tag for all of them.  The
 * indices stay on the device (the routing output of fmoe_route_topk feeds it
 * directly), and repeated experts are copied once.
 *   idx [n_idx] int32 DEVICE (entries outside [0, n_slots) copy nothing),
 *   n_idx <= 8192; host_slabs: pinned host memory mapped for the GPU (for
 *   example hipHostMalloc or a pinned torch tensor), n_slots slabs of
 *   slab_stride bytes (FMOE_ERR_UNSUPPORTED if the pointer is not pinned host
 *   memory); dev_slabs: device memory, the same layout; tags [n_slots] int32
 *   DEVICE; n_copied: optional int32 DEVICE counter incremented once per slab
 *   copied.  slab_bytes a positive multiple of 16 <= slab_stride, a multiple of
 *   16; both base pointers 16-byte aligned.  Two calls whose fetch lists share
 *   an expert must not run concurrently. */
fmoe_status fmoe_fetch_experts(const int32_t *idx, int32_t n_idx, int32_t shared,
                               const void *host_slabs, int64_t slab_bytes, int64_t slab_stride,
                               void *dev_slabs, int32_t *tags, int32_t n_slots, int32_t tag,
                               int32_t *n_copied, void *stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): fmoe_moe_layer_forward with
 * the same arguments and results, minus the workspace.  Its workspace is a
 * static device array of FMOE_STATIC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends; the call allocates nothing.
 *   - A layer that needs more than that (fmoe_workspace_size(L, T) >
 *     FMOE_STATIC_SCRATCH_BYTES; T up to about 110 at hidden 4096 / inter 1024
 *     / 512 experts) returns FMOE_ERR_WORKSPACE and enqueues nothing.
 *   - The first call on each device takes the array's address and clears it
 *     on `stream`; that first call must not be under graph capture
 *     (FMOE_ERR_HIP otherwise).  Later calls may be captured.
 *   - Every call on one GPU shares that GPU's array: calls whose execution
 *     overlaps (other streams, other threads) race and give undefined results.
 *     Calls in one stream are ordered and safe.
 *   - A bounded in-kernel wait that gives up leaves NaN outputs (the timeout
 *     word lives in the array and is not reachable by the caller). */
#define FMOE_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
fmoe_status fmoe_moe_layer_forward_noalloc(const fmoe_layer *L, int32_t T, const float *x,
                                           const float *residual, float *h_out, float *y_out,
                                           int32_t *idx_out, float *w_out, float *moe_out,
                                           void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FMOE_H */
