/*
 * pvj.h -- C ABI of libpvj: packed variable-length joint text+image attention
 * with per-sample 2D RoPE, for AMD Instinct MI355X (gfx950).
 *
 * What it computes (Mage-Flow pages):
 *  - Mage-Flow review page (startedourmission.github.io), section
 *    "Native-Resolution MMDiT": images of different resolutions become
 *    variable-length latent token sequences, which are packed with their text
 *    conditions (no padding) into one contiguous batch; per-sample cumulative
 *    offsets confine attention to each sample without a block-diagonal mask;
 *    text and image tokens of a sample are concatenated and processed by joint
 *    self-attention; classifier-free guidance's conditional and unconditional
 *    branches share one pack and one forward.
 *  - same page, section "Mage-VAE": one latent token per 16x16 pixels.
 *  - Hugging Face paper page (arXiv 2607.19064), "Highlights", and the model
 *    card "microsoft/Mage-Flow", section "Architecture": per-sample 2D rotary
 *    embeddings on the packed image+text sequence.
 *  - Hugging Face model card, section "Python API": per-sample resolutions are
 *    batched into one packed forward per denoising step.
 *
 * Conventions the pages leave open (fixed here, identical in every entry point):
 *  - a sample is (h_lat, w_lat, l_text); its L = l_text + h_lat*w_lat tokens
 *    are packed text first, then the image grid row-major; samples keep their
 *    input order; T = sum of L over samples;
 *  - RoPE position of text tokens is (0,0) (no rotation); image token p of a
 *    sample sits at (p / w_lat, p % w_lat);
 *  - 2D RoPE: dims [0, D/2) rotate by the row, [D/2, D) by the column; pair k
 *    of an axis is dims (base+2k, base+2k+1) with angle pos*theta^(-k/(D/4));
 *    (a,b) -> (a cos - b sin, a sin + b cos); V is never rotated;
 *  - attention is non-causal; softmax_scale <= 0 selects 1/sqrt(D).
 *
 * Layout and ownership:
 *  - every token tensor is contiguous row-major [T, H, D] (token stride H*D,
 *    head stride D) in the plan's dtype; LSE is fp32 [H, T] (natural log);
 *    base pointers must be 16-byte aligned; all are device pointers;
 *  - the caller allocates and owns all device memory (tensors, LSE, the
 *    metadata buffer, the backward workspace); the library allocates only host
 *    memory (the plan);
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream); all
 *    device work is enqueued asynchronously on it; no entry point synchronises.
 *
 * Errors: every call returns a status; arguments are validated before anything
 * is enqueued, so a failing call leaves the stream untouched.  A launch error
 * reported by the HIP runtime maps to PVJ_ERR_HIP.  pvj_last_error() gives a
 * human-readable detail of the last failure on the calling thread.
 */
#ifndef PVJ_H
#define PVJ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PVJ_API __attribute__((visibility("default")))

typedef enum pvj_status {
  PVJ_OK = 0,
  PVJ_ERR_INVALID_ARG = 1,         /* null/misaligned pointer, negative size, bad enum */
  PVJ_ERR_UNSUPPORTED = 2,         /* head_dim not in {64,128}, unsupported dtype/pairing,
                                      latent side above 32767 */
  PVJ_ERR_OVERFLOW = 3,            /* T or a per-sample length does not fit int32 */
  PVJ_ERR_NOT_UPLOADED = 4,        /* compute call before pvj_plan_upload */
  PVJ_ERR_WORKSPACE_TOO_SMALL = 5, /* workspace / metadata buffer smaller than required */
  PVJ_ERR_HIP = 6                  /* the HIP runtime reported an error */
} pvj_status_t;

enum { PVJ_BF16 = 0, PVJ_F32 = 1 };          /* pvj_plan_desc_t.dtype */
enum { PVJ_ROPE_INTERLEAVED = 0 };           /* pvj_plan_desc_t.rope_pairing */
enum { PVJ_FLAG_ROPE_FUSED = 1u,             /* attention flags */
       PVJ_FLAG_ROPE_PREROTATED = 2u,        /* backward only */
       PVJ_FLAG_STREAM_MAJOR = 4u };         /* token tensors in stream-major order (see
                                                pvj_rope2d_apply_stream_major) */

typedef struct pvj_sample {
  int32_t h_lat;  /* latent rows    (image pixels / 16), 0 .. 32767 */
  int32_t w_lat;  /* latent columns (image pixels / 16), 0 .. 32767 */
  int32_t l_text; /* text tokens, >= 0 */
} pvj_sample_t;

/* An editing sample: n_frames latent grids of h_lat x w_lat (source, target,
 * ...) after its l_text text tokens, frame after frame, each row-major. */
typedef struct pvj_sample_frames {
  int32_t h_lat;    /* 0 .. 32767 */
  int32_t w_lat;    /* 0 .. 32767 */
  int32_t l_text;   /* >= 0 */
  int32_t n_frames; /* 0 .. 32767 */
} pvj_sample_frames_t;

typedef struct pvj_plan_desc {
  int32_t n_heads;      /* H >= 1 */
  int32_t head_dim;     /* D in {64, 128} */
  int32_t dtype;        /* PVJ_BF16 or PVJ_F32: element type of every token tensor */
  float rope_theta;     /* RoPE base, > 0 (10000) */
  int32_t rope_pairing; /* PVJ_ROPE_INTERLEAVED */
  int32_t text_first;   /* must be 1: text tokens precede image tokens in a sample */
} pvj_plan_desc_t;

typedef struct pvj_plan pvj_plan_t;

/* ---- plan (pure host) -------------------------------------------------------
 * pvj_plan_create: build the per-pack plan from the per-sample latent sizes
 * (HF model card, "Python API": each sample its own resolution, one packed
 * forward per step; review page, "Native-Resolution MMDiT": per-sample
 * cumulative offsets).  It computes cu_seqlens (int32 [B+1], cu[0]=0,
 * cu[i+1]=cu[i]+L_i), the per-sample metadata, the RoPE cos/sin tables (fp64
 * math rounded to fp32) and the attention work lists (largest samples first,
 * (sample, head) groups kept together and spread over the 8 XCDs).
 * Zero-length samples are allowed.  n_samples may be 0.
 * On success *out owns a new plan; free it with pvj_plan_destroy.
 */
PVJ_API pvj_status_t pvj_plan_create(const pvj_sample_t* samples, int32_t n_samples,
                                     const pvj_plan_desc_t* desc, pvj_plan_t** out);

/* Editing packs (review page, "Native-Resolution MMDiT": the edit model adds a
 * frame axis to the 2D RoPE, so each visual token carries an (h, w, f) index
 * that tells source from target tokens).  Like pvj_plan_create, but sample i
 * has l_text + n_frames*h_lat*w_lat tokens, and every RoPE of the plan (the
 * standalone apply, the fused attention loads, the backward's inverse) is
 * 3-axis: text at (0,0,0); image token p at (row, col, frame) =
 * ((p mod hw) / w, p mod w, p / hw); the head dim is split into consecutive
 * row | col | frame parts of (D-16)/2, (D-16)/2 and 16 dims, each a 1D rotary
 * embedding of its own dimension d_a (pair k turns by pos * theta^(-k/(d_a/2))).
 * The pack streams hold the text rows and all frames' image rows. */
PVJ_API pvj_status_t pvj_plan_create_frames(const pvj_sample_frames_t* samples, int32_t n_samples,
                                            const pvj_plan_desc_t* desc, pvj_plan_t** out);

/* Sizes of a plan.  Any output pointer may be NULL.  *cu_seqlens_host points
 * into the plan (B+1 int32, valid until destroy); *meta_bytes is the size of
 * the device metadata buffer pvj_plan_upload needs: the metadata itself, then
 * (bf16 plans with samples of 1,985 to 8,192 tokens) the partial-result slots
 * of the forward's split query tiles, (head_dim + 2) * 256 * 4 bytes each (see
 * pvj_varlen_attn_fwd). */
PVJ_API pvj_status_t pvj_plan_info(const pvj_plan_t* plan, int64_t* n_tokens, int32_t* max_len,
                                   const int32_t** cu_seqlens_host, size_t* meta_bytes);

/* Rows of the two modality streams of a plan: *n_text = sum of l_text, *n_image
 * = sum of n_frames*h_lat*w_lat (review page, "Native-Resolution MMDiT": text
 * and image keep separate streams around the joint attention).  Either output
 * may be NULL. */
PVJ_API pvj_status_t pvj_plan_streams(const pvj_plan_t* plan, int64_t* n_text, int64_t* n_image);

/* The stream-major row of every token (see PVJ_FLAG_STREAM_MAJOR below): for
 * the joint row t (sample i's local token j), rows[t] = the row of the same
 * token when all samples' text rows come first and then all image rows, each
 * in sample order.  rows: host int32 array of n = T entries, owned by the
 * caller (n != T or rows NULL with T > 0: INVALID_ARG).  Pure host. */
PVJ_API pvj_status_t pvj_plan_stream_major_rows(const pvj_plan_t* plan, int32_t* rows, int64_t n);

/* Copy the plan's metadata into the caller-allocated device buffer `dev_meta`
 * (>= meta_bytes, 256-byte aligned) on `stream`, and record it in the plan.
 * Compute calls on this plan then read that buffer (and the forward writes its
 * partial-result slots, which are not uploaded and need no initialisation); it
 * must stay allocated and otherwise unmodified while they run.  Calling it
 * again re-targets the plan. */
PVJ_API pvj_status_t pvj_plan_upload(pvj_plan_t* plan, void* dev_meta, size_t bytes, void* stream);

/* Free the plan (host memory only).  Work already enqueued that uses the plan's
 * device metadata is unaffected (the caller owns that buffer). */
PVJ_API void pvj_plan_destroy(pvj_plan_t* plan);

/* ---- the two modality streams ----------------------------------------------
 * Review page, "Native-Resolution MMDiT": modality-specific layers keep text
 * and image as two streams; their tokens are concatenated per sample for the
 * joint attention.  text is [sum l_text, H, D], image [sum h*w, H, D], each
 * stream packed in sample order without padding; joint is [T, H, D] with
 * sample i's rows [text_i ; image_i].  pvj_unpack is the exact inverse.
 * Buffers must not overlap.  Pure data movement (bit-exact).
 */
PVJ_API pvj_status_t pvj_pack(const pvj_plan_t* plan, const void* text, const void* image,
                              void* joint, void* stream);
PVJ_API pvj_status_t pvj_unpack(const pvj_plan_t* plan, const void* joint, void* text,
                                void* image, void* stream);

/* Pack or unpack with the RoPE in the same pass (review page, "Kernel fusion":
 * the memory-bound chains, RoPE application among them, are fused so each
 * tensor is read and written once).  pvj_pack_rope writes R(pos) x (inverse
 * != 0: R(pos)^T x) into the joint layout; pvj_unpack_rope rotates each joint
 * row before scattering it to the streams.  The result is bitwise that of
 * pvj_pack then pvj_rope2d_apply (or pvj_rope2d_apply then pvj_unpack): fp32
 * rotation from the plan's tables, rounded once to the plan dtype.  Q and K
 * packed this way feed pvj_varlen_attn_fwd without flags and
 * pvj_varlen_attn_bwd with PVJ_FLAG_ROPE_PREROTATED.  Buffers must not
 * overlap. */
PVJ_API pvj_status_t pvj_pack_rope(const pvj_plan_t* plan, const void* text, const void* image,
                                   void* joint, int32_t inverse, void* stream);
PVJ_API pvj_status_t pvj_unpack_rope(const pvj_plan_t* plan, const void* joint, void* text,
                                     void* image, int32_t inverse, void* stream);

/* ---- standalone per-sample 2D RoPE ------------------------------------------
 * HF paper page "Highlights" / model card "Architecture": per-sample 2D rotary
 * embedding; review page, "Kernel fusion": RoPE application is one of the
 * memory-bound ops.  y = R(pos) x on [T, H, D] (inverse != 0: y = R(pos)^T x).
 * x == y (in place) is allowed; otherwise the buffers must not overlap.
 * Computed in fp32 from the plan's tables, rounded once to the output dtype.
 */
PVJ_API pvj_status_t pvj_rope2d_apply(const pvj_plan_t* plan, const void* x, void* y,
                                      int32_t inverse, void* stream);

/* ---- stream-major layout -------------------------------------------------------
 * Review page, "Native-Resolution MMDiT": the modality-specific layers keep
 * text and image as two streams, and only the joint attention sees a sample's
 * text and image tokens together; "Kernel fusion": each tensor of the
 * memory-bound work is read and written once.  A stream-major token tensor is
 * [T, H, D] holding the text stream's n_text rows (sample order) and then the
 * image stream's n_image rows: the two stream tensors of pvj_pack placed one
 * after the other in one allocation.  With PVJ_FLAG_STREAM_MAJOR the attention
 * calls read and write every token tensor (q, k, v, o, dout, dq, dk, dv) in
 * this layout and index LSE [H, T] (and the backward's Delta) by the same row
 * order, so the streams' projections feed the attention, and take its output,
 * with no pack or unpack pass.  Each sample still attends over its own text
 * and image tokens only, in the order text then image, and every value is
 * bitwise what the joint layout gives for the same rows (the kernels and the
 * order of every sum are the same; only the row addresses differ).
 * Conditions (else UNSUPPORTED, before anything is enqueued): a bf16 plan; no
 * PVJ_FLAG_ROPE_FUSED (rotate Q and K with pvj_rope2d_apply_stream_major, call
 * the forward without RoPE flags and the backward with
 * PVJ_FLAG_ROPE_PREROTATED); (T + 256) * H * D * 2 < 2^31 (32-bit row
 * offsets).
 * pvj_rope2d_apply_stream_major: pvj_rope2d_apply for a stream-major x, y
 * (each row rotated by its own token's position; bitwise the same values as
 * the joint-layout call; any plan dtype; x == y allowed, else no overlap).
 */
PVJ_API pvj_status_t pvj_rope2d_apply_stream_major(const pvj_plan_t* plan, const void* x,
                                                   void* y, int32_t inverse, void* stream);

/* ---- attention forward -------------------------------------------------------
 * For every sample i and head h: O_i = softmax(s * Q'_i K'_i^T) V_i over the
 * sample's own L_i keys only (review page, "Native-Resolution MMDiT": joint
 * self-attention confined by per-sample offsets), with Q' = R Q, K' = R K when
 * flags has PVJ_FLAG_ROPE_FUSED (the rotation is applied on load) and Q' = Q,
 * K' = K otherwise.  lse[h, t] = log sum_j exp(s q'_t . k'_j) (natural log,
 * fp32; may be NULL if not needed).  bf16 inputs use bf16 matrix cores with
 * fp32 accumulation and fp32 online softmax; fp32 inputs use fp32 matrix cores.
 * o must not overlap q, k, v.  Deterministic: the same inputs give the same
 * bits, and a sample's result does not depend on the rest of the pack.
 * Work split (bf16 plans): the last 256-query tile of each (sample, head) of a
 * sample of 1,985 to 8,192 tokens (32 to 128 tiles of 64 keys) is computed as
 * min(4, floor(tiles / 16)) ranges of its keys (a function of the sample
 * length only) whose partial softmax states go to the
 * plan buffer's slots and are merged in a fixed order by a second kernel on
 * the same stream; so two forward calls on one uploaded plan must not run at
 * the same time (on different streams).
 * flags: PVJ_FLAG_ROPE_FUSED, PVJ_FLAG_STREAM_MAJOR (token tensors and LSE's
 * columns in the stream-major row order, above); others are INVALID_ARG.
 */
PVJ_API pvj_status_t pvj_varlen_attn_fwd(const pvj_plan_t* plan, const void* q, const void* k,
                                         const void* v, void* o, float* lse,
                                         float softmax_scale, uint32_t flags, void* stream);

/* ---- attention backward ------------------------------------------------------
 * Gradients of sum(O * dO) (training uses forward + backward; review page,
 * "Kernel fusion": 8-GPU training at ~50K packed tokens per GPU):
 *   Delta = rowsum(dO * O); P = exp(s Q'K'^T - LSE); dV = P^T dO;
 *   dS = P * (dO V^T - Delta); dQ' = s dS K'; dK' = s dS^T Q';
 * with PVJ_FLAG_ROPE_FUSED, Q' = R Q and K' = R K are formed here and
 * dQ = R^T dQ', dK = R^T dK' (gradients with respect to the un-rotated Q, K);
 * with PVJ_FLAG_ROPE_PREROTATED, q and k already hold Q' and K' (for example
 * from pvj_pack_rope, with a forward called without flags) and dQ = R^T dQ',
 * dK = R^T dK' likewise; with neither, dQ = dQ', dK = dK'.  The two flags
 * exclude each other (INVALID_ARG).  Both RoPE modes give the same bits when
 * the pre-rotated Q', K' were rounded as pvj_rope2d_apply rounds them.
 * q, k, v, o, lse and the scale must be those of the forward call.
 * workspace: device memory of at least pvj_varlen_attn_bwd_workspace bytes,
 * 256-byte aligned, owned by the caller, contents need not be initialised;
 * it holds Delta (fp32 [H, T]) and, with PVJ_FLAG_ROPE_FUSED, the rotated
 * Q' and K' (two [T, H, D] tensors in the plan dtype; the size always counts
 * them).  No atomics: dQ, dK
 * and dV are deterministic (the same inputs give the same bits).  Enqueued
 * as: (RoPE on load only) the rotation of Q and K, the dQ pass, which also
 * forms Delta, then the dK/dV pass.  PVJ_FLAG_STREAM_MAJOR as in the forward.
 */
PVJ_API pvj_status_t pvj_varlen_attn_bwd_workspace(const pvj_plan_t* plan, size_t* bytes);
PVJ_API pvj_status_t pvj_varlen_attn_bwd(const pvj_plan_t* plan, const void* q, const void* k,
                                         const void* v, const void* o, const float* lse,
                                         const void* dout, void* dq, void* dk, void* dv,
                                         void* workspace, size_t ws_bytes, float softmax_scale,
                                         uint32_t flags, void* stream);

/* ---- attention backward without device allocation -----------------------------
 * For callers that cannot allocate device memory or pass a workspace (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Computes exactly what pvj_varlen_attn_bwd computes, with the
 * same kernels and the same bits, but its scratch buffer (Delta, fp32 [H, T])
 * lives in a static device array the library owns: PVJ_NOALLOC_SCRATCH_BYTES
 * per GPU, held from the library's first use on that GPU until the process
 * ends.  Limits, checked before anything is enqueued:
 *  - align256(H * T * 4) <= PVJ_NOALLOC_SCRATCH_BYTES (16 MiB: H * T up to
 *    4,194,304, e.g. 24 heads x 174,762 tokens), else WORKSPACE_TOO_SMALL;
 *  - PVJ_FLAG_ROPE_FUSED is UNSUPPORTED (its rotated Q', K' would not fit);
 *    pass Q, K pre-rotated (pvj_pack_rope) with PVJ_FLAG_ROPE_PREROTATED.
 * The caller still owns q, k, v, o, lse, dout and the outputs dq, dk, dv.
 * Nothing is allocated or freed (device or pinned host memory).  Every call on
 * one GPU shares that GPU's scratch array: calls that overlap in time on one
 * GPU (several streams or host threads) race and must be serialised by the
 * caller; calls in order on one stream are safe.  The array keeps the last
 * call's contents; nothing in it needs clearing between calls.
 */
#define PVJ_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
PVJ_API pvj_status_t pvj_varlen_attn_bwd_noalloc(const pvj_plan_t* plan, const void* q,
                                                 const void* k, const void* v, const void* o,
                                                 const float* lse, const void* dout, void* dq,
                                                 void* dk, void* dv, float softmax_scale,
                                                 uint32_t flags, void* stream);

/* ---- memory-bound chains around the attention ---------------------------------
 * Review page, "Kernel fusion": the backbone's memory-bound chains
 * (normalization, adaptive modulation, gating, residual addition) are fused so
 * each tensor is read and written once; "Native-Resolution MMDiT": the text
 * and image streams keep modality-specific parameters.  Reading taken (the
 * pages name the operations, not the formulas): adaptive LayerNorm of the
 * MMDiT block design, LayerNorm without affine parameters, population
 * variance.
 *
 * Every call works on one stream of the plan (which = PVJ_STREAM_TEXT: the
 * n_text rows in sample order; PVJ_STREAM_IMAGE: the n_image rows) with
 * `hidden` columns (a multiple of 8 in [8, 8192]).  Row tensors are
 * [rows, hidden] and per-sample vectors [n_samples, hidden], in the plan
 * dtype, row-major, 16-byte aligned; a row's sample is the one whose slice of
 * the stream holds it.  Parameter gradients are fp32 [n_samples, hidden]
 * (zero for samples without rows in the stream).  Computation is fp32.
 * Deterministic: the per-sample sums are reduced in a fixed order.
 *
 * which = PVJ_STREAM_BOTH runs both streams in one call: row tensors are
 * [n_text + n_image, hidden], the text stream's rows and then the image
 * stream's (the stream-major row order above, at the model width), and every
 * per-sample vector and parameter gradient is [2, n_samples, hidden], the
 * text stream's parameters first.  Rows, and so y, out, dx and dy, get the
 * same bits as the two one-stream calls; the parameter gradients add the same
 * terms in another fixed order (the per-sample slots are cut from the joint
 * row count), so they agree with the one-stream calls to fp32 rounding.
 */
enum { PVJ_STREAM_TEXT = 0, PVJ_STREAM_IMAGE = 1, PVJ_STREAM_BOTH = 2 };
enum { PVJ_CHAIN_ADALN = 0, PVJ_CHAIN_GATE = 1 };

/* y = LN(x) * (1 + scale_i) + shift_i, LN over hidden with `eps` (1e-6).
 * y may equal x (in place). */
PVJ_API pvj_status_t pvj_adaln_modulate(const pvj_plan_t* plan, int32_t which, int32_t hidden,
                                        const void* x, const void* shift, const void* scale,
                                        void* y, float eps, void* stream);
/* out = x + gate_i * y.  out may equal x or y. */
PVJ_API pvj_status_t pvj_gate_residual(const pvj_plan_t* plan, int32_t which, int32_t hidden,
                                       const void* x, const void* y, const void* gate, void* out,
                                       void* stream);
/* Workspace of a chain backward (op = PVJ_CHAIN_ADALN or PVJ_CHAIN_GATE) on
 * stream `which` (PVJ_STREAM_BOTH included): per-sample partial sums, and for
 * the layer norm the row statistics. */
PVJ_API pvj_status_t pvj_chain_bwd_workspace(const pvj_plan_t* plan, int32_t op, int32_t which,
                                             int32_t hidden, size_t* bytes);
/* Gradients of sum(y * dy): dx (plan dtype, rows x hidden), dshift_i = sum of
 * dy over the sample's rows, dscale_i = sum of dy * xhat; x, scale and eps
 * are those of the forward.  dx must not overlap x or dy. */
PVJ_API pvj_status_t pvj_adaln_modulate_bwd(const pvj_plan_t* plan, int32_t which, int32_t hidden,
                                            const void* x, const void* scale, const void* dy,
                                            void* dx, float* dshift, float* dscale, float eps,
                                            void* workspace, size_t ws_bytes, void* stream);
/* Gradients of sum(out * dout): dy = gate_i * dout, dgate_i = sum over the
 * sample's rows of dout * y; the gradient of x is dout itself (no copy made).
 * dy must not overlap y or dout. */
PVJ_API pvj_status_t pvj_gate_residual_bwd(const pvj_plan_t* plan, int32_t which, int32_t hidden,
                                           const void* y, const void* gate, const void* dout,
                                           void* dy, float* dgate, void* workspace,
                                           size_t ws_bytes, void* stream);

/* ---- introspection (pure host; used by tests and tooling) -------------------- */

/* Attention work list of the plan: which = 0 forward, 1 backward dK/dV, 2
 * backward dQ (the forward's query tiles, none split), 3 the forward's split
 * tiles.  *items points to n_items int32 quadruples {sample, head, tile,
 * split} in launch order (sample = -1 marks an idle slot); split = 0 for a
 * whole tile, else bits 0-3 = parts - 1, bits 4-7 = this part (lists 0), bits
 * 8-31 = the tile's first partial-result slot; part j of n covers key tiles
 * [nkt j / n, nkt (j + 1) / n) of 64 keys, nkt = ceil(L / 64).  *tile_rows is
 * the rows of one tile (query rows forward and dQ, key rows dK/dV).  Valid
 * until destroy. */
PVJ_API pvj_status_t pvj_plan_work_items(const pvj_plan_t* plan, int32_t which,
                                         const int32_t** items, int32_t* n_items,
                                         int32_t* tile_rows);

/* RoPE tables: cos/sin[p * n_pairs + k] for position p in [0, n_pos) and head-dim
 * pair k (dims 2k, 2k+1) in [0, n_pairs = D/2): cos/sin(p * theta^(-j/(d_a/2)))
 * where pair k is pair j of its axis part a (of d_a dims), fp64 rounded to
 * fp32.  Valid until destroy. */
PVJ_API pvj_status_t pvj_plan_rope_table(const pvj_plan_t* plan, const float** cos_tab,
                                         const float** sin_tab, int32_t* n_pos, int32_t* n_pairs);
/* RoPE axes of the plan: n_axes = 2 (row, col) or 3 (row, col, frame) and the
 * head-dim size of each part (dims[2] = 0 for two axes). */
PVJ_API pvj_status_t pvj_plan_rope_axes(const pvj_plan_t* plan, int32_t* n_axes, int32_t dims[3]);

/* ---- projections with the modality pack / unpack fused in -----------------------
 * Review page, "Native-Resolution MMDiT": each modality stream has its own
 * projection layers; the tokens are concatenated only for the joint attention.
 * Reading taken (the pages do not write the layer out): a linear layer with
 * bias per stream, y = x W^T + b, W row-major [out_features, in_features] (the
 * usual layout of a linear layer's weight), the QKV output ordered [Q | K | V]
 * along the features and each part [H, D].  bf16 plans only; fp32
 * accumulation, one rounding of each output.  hidden is a multiple of 64 in
 * [64, 65536]; bias may be NULL.
 *
 * pvj_qkv_proj_pack: for the rows of one stream (x [rows, hidden], w
 * [3 H D, hidden], bias [3 H D]) writes each token's Q, K and V straight into
 * its joint row of q, k, v ([T, H, D]); with PVJ_FLAG_ROPE_FUSED the plan's
 * RoPE is applied to Q and K before the rounding (the values pvj_pack_rope
 * would produce from the projected streams, up to that rounding).  Calling it
 * for both streams fills every joint row.
 * pvj_out_proj_unpack: y [rows, hidden] = o_s W^T + b, where o_s are the
 * stream's rows of the joint o [T, H, D] (w [hidden, H D], bias [hidden]).
 */
PVJ_API pvj_status_t pvj_qkv_proj_pack(const pvj_plan_t* plan, int32_t which, int32_t hidden,
                                       const void* x, const void* w, const void* bias, void* q,
                                       void* k, void* v, uint32_t flags, void* stream);
PVJ_API pvj_status_t pvj_out_proj_unpack(const pvj_plan_t* plan, int32_t which, int32_t hidden,
                                         const void* o, const void* w, const void* bias, void* y,
                                         void* stream);

/* ---- diagnostic: measured matrix-core ceiling -----------------------------------
 * Enqueues a kernel that keeps every SIMD issuing only independent
 * v_mfma_f32_32x32x16_bf16 (2 workgroups of 4 waves per CU, `rounds` times
 * over the 256 CUs, `iters` x 4 products per wave) and returns its bf16 FLOP
 * count in *flop; timing it (events on `stream`) gives the sustained
 * matrix-core rate the attention kernels are compared with beside the
 * published dense peak.  sink: device fp32, >= 131072 * rounds floats
 * (receives the accumulators so the work is kept). */
PVJ_API pvj_status_t pvj_diag_mfma_peak(int32_t rounds, int32_t iters, float* sink,
                                        size_t sink_floats, double* flop, void* stream);

/* ---- per-kernel timing (tracing) ---------------------------------------------
 * When enabled, every kernel the library launches is bracketed by two HIP
 * events recorded on the stream it is launched on; pvj_profile_read waits for
 * the recorded events of one kernel kind and returns their summed duration and
 * count since the last enable.  Disabled by default (no events, no overhead).
 * pvj_profile_enable(1) clears the record; (0) stops recording.  Not
 * thread-safe against concurrent launches from several host threads. */
enum {
  PVJ_KERNEL_PACK = 0,
  PVJ_KERNEL_UNPACK = 1,
  PVJ_KERNEL_ROPE = 2,
  PVJ_KERNEL_ATTN_FWD = 3,
  PVJ_KERNEL_BWD_PRE = 4,          /* the backward's rotation of Q, K (RoPE on load only) */
  PVJ_KERNEL_ATTN_BWD = 5,         /* dK, dV */
  PVJ_KERNEL_ATTN_BWD_DQ = 6,      /* dQ and Delta */
  PVJ_KERNEL_CHAIN_FWD = 7,        /* adaptive layer norm, gate + residual */
  PVJ_KERNEL_CHAIN_BWD = 8,        /* their backward passes */
  PVJ_KERNEL_PROJ = 9,             /* projections with the pack / unpack fused */
  PVJ_KERNEL_COUNT = 10
};
PVJ_API pvj_status_t pvj_profile_enable(int32_t on);
PVJ_API pvj_status_t pvj_profile_read(int32_t kernel, double* total_ms, int64_t* launches);

PVJ_API const char* pvj_status_string(pvj_status_t status);
PVJ_API const char* pvj_last_error(void);
PVJ_API const char* pvj_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PVJ_H */
