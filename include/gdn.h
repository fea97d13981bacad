/*
 * gdn.h -- C ABI of the MI355X (gfx950) frame-wise Gated DeltaNet: the forward
 * (whole sequence and streaming chunks), its backward, and the two companion
 * operations of the hybrid model (the block-causal temporal convolution of the
 * streaming FFN, the block-causal softmax attention blocks).
 *
 * What is computed.  SANA-WM's frame-wise GDN ("NVIDIA Apresenta SANA-WM ...",
 * acheiumaia.com.br, section "1. Atencao Linear Hibrida com Gated DeltaNet
 * (GDN)"; also the hybrid GDN + softmax design named in the abstract of
 * "SANA-WM: Efficient Minute-Scale World Modeling with Hybrid Linear Diffusion
 * Transformer"): every head carries a constant D x D state M[key][value] across
 * latent frames; one recurrent step consumes a whole frame of S tokens:
 *
 *   Qf = ReLU(Q_t),  Kf = ReLU(K_t) / sqrt(D*S)
 *   Md = gamma_t * M                                  (decay gate)
 *   R  = V_t - beta_t * Kf Md        (ERASE)          (delta-rule residual)
 *   R  = beta_t * (V_t - Kf Md)      (WRITE)
 *   M  = Md + Kf^T R                                  (write)
 *   O_t = Qf M                                        (readout, post-update)
 *
 * ERASE with beta = 0 and gamma = 1 is SANA-Video's cumulative ReLU linear
 * attention (the block KV-cache of the talk "SANA-Video: Efficient Video
 * Generation with Block Linear Diffusion Transformer"); WRITE with S = 1 is
 * the token-wise gated delta rule.  gamma and beta are already activated
 * fp32 scalars, one per (batch, head, frame).
 *
 * Layouts (all row-major, innermost last; every pointer is a DEVICE pointer):
 *   q, k, v, o     [B][H][T][S][D]  io_dtype (bf16, fp32 or OCP e4m3)
 *   gamma, beta    [B][H][T]        fp32
 *   state_in/out   [B][H][D][D]     fp32, indexed [key][value]
 *   state_norms    [B][H][T]        fp32, Frobenius norm of the post-update state
 *
 * Conventions.
 *   - Ownership: the caller owns every buffer.  The library never allocates
 *     device memory; scratch space comes in through `workspace`.
 *   - Streams: every call enqueues work and returns without synchronising;
 *     `stream` is a hipStream_t (NULL = the default stream).  Device faults
 *     surface at the caller's next synchronisation.  The bf16/e4m3 forward,
 *     the training pair and the backward also run part of their kernels on
 *     a side stream of the library's own: one non-blocking stream at default
 *     priority per (host thread, device), created on the thread's first such
 *     call and released when the thread exits.  Its work starts after
 *     everything enqueued on `stream` before the call and is finished before
 *     anything enqueued on `stream` after the call returns (event waits on
 *     both sides), so the call behaves as if it ran on `stream` alone.  Two
 *     calls on different caller streams from one host thread share that side
 *     stream, which orders their side-stream parts one after the other.
 *   - Errors: arguments are checked on the host before anything is launched;
 *     a failing check returns a status and launches nothing.  The library
 *     never aborts.  gdn_last_error() gives a per-thread message.
 *   - Aliasing: o must not overlap q, k, v, gamma, beta, the states or the
 *     workspace.  state_out may equal state_in exactly (in-place update) but
 *     may not partially overlap it.
 *   - Alignment: q, k, v, o 16-byte aligned; gamma, beta, states, norms 4-byte
 *     aligned; workspace 256-byte aligned.
 *   - Shapes: B, H, T, S >= 1; D in {16, 32, 48, ..., 128}; one head's q (and
 *     k, v, o) must stay below 2 GiB, T*S*D*element_size < 2^31 (the kernels
 *     address a head with 32-bit byte offsets).
 *   - Determinism: results do not depend on the workspace size or on how the
 *     frames are split across calls; the same inputs and flags give the same
 *     bits.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 1

/*
 * Element type of q, k, v and o.  GDN_FP8_E4M3 is the OCP 8-bit float E4M3
 * ("fn": exponent bias 7, no infinities, 0x7F/0xFF NaN), a low-precision I/O
 * variant of the same computation (after the 4-bit NVFP4 deployment the
 * SANA-WM news article describes): inputs are decoded exactly, the Gram
 * pipeline runs as for bf16, and o is rounded once from fp32 to the nearest
 * e4m3 (ties to even; magnitudes past 448's rounding range become NaN).
 */
typedef enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1, GDN_FP8_E4M3 = 2 } gdn_dtype;

typedef enum gdn_beta_mode {
  GDN_BETA_ERASE = 0, /* M = gM + Kf^T (V - b Kf gM): beta scales the correction */
  GDN_BETA_WRITE = 1  /* M = gM + b Kf^T (V - Kf gM): beta scales the written residual */
} gdn_beta_mode;

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_NULL = 1,        /* a required pointer is NULL */
  GDN_ERR_SHAPE = 2,       /* B, H, T or S out of range, or sizes overflow */
  GDN_ERR_DTYPE = 3,       /* io_dtype or beta_mode not one of the enums */
  GDN_ERR_ALIGN = 4,       /* a pointer is not aligned as required */
  GDN_ERR_ALIAS = 5,       /* forbidden overlap between buffers */
  GDN_ERR_UNSUPPORTED = 6, /* D not in {16, 32, ..., 128}, unknown flags, or DIRECT with e4m3 */
  GDN_ERR_ABI = 7,         /* desc->abi_version != GDN_ABI_VERSION */
  GDN_ERR_WORKSPACE = 8,   /* workspace NULL or smaller than one frame needs */
  GDN_ERR_HIP = 9          /* a HIP runtime call failed (message in gdn_last_error) */
} gdn_status;

/* Record device time per kernel on `stream` (read back with gdn_kernel_times). */
#define GDN_FLAG_TIME_KERNELS 0x1u
/*
 * bf16 I/O only (GDN_ERR_UNSUPPORTED with e4m3): run the single-pass recurrence (keys and values streamed by
 * every value-column tile of the state, the state product in the same sweep)
 * instead of the default Gram pipeline (frame-parallel G_t = Kf^T Kf and
 * B_t = Kf^T V, then a serial D x D state pass).  Slower; needs no G/B
 * staging in the workspace.  The two agree to rounding, not bitwise.  fp32 I/O
 * always runs the single-pass recurrence.
 */
#define GDN_FLAG_DIRECT 0x2u
/*
 * bf16/e4m3 I/O, the two forms of the Gram pipeline.  Three launches: gram
 * pass, state pass, readout; G_t, B_t and the bf16 states go through the
 * workspace in HBM.  One launch: the three roles in one persistent kernel,
 * every head on one XCD, those per-frame terms handed over in that XCD's L2.
 * Both compute the same operations in the same order: the results are
 * bitwise equal.  By default calls with B*H*T*S*D >= 2^26 (bf16) or
 * >= 2^28 (e4m3) take the one launch (it needs a cooperative launch, at most
 * 16 XCDs, every XCD's workgroups at least twice its heads' chain
 * workgroups, and the workspace gdn_workspace_size gives), the rest the
 * three.  Of the rest, a short call -- at most 4 frames per head, D <= 112,
 * B*H*T no more than the device's compute units, state_norms NULL, the
 * whole call in one range of the workspace (a streaming chunk) -- runs the
 * state pass and the readout as one kernel, each of its workgroups
 * recomputing the state chain of the frames before its own: two launches,
 * the same bits.  GDN_FLAG_THREE_PASS forces the three launches;
 * GDN_FLAG_ONE_LAUNCH asks for the one launch whatever the size or dtype (it
 * still falls back where the device or the workspace does not allow it).  The
 * two flags exclude each other.
 */
#define GDN_FLAG_THREE_PASS 0x4u
#define GDN_FLAG_ONE_LAUNCH 0x8u

/* Kernel kinds booked by gdn_kernel_times. */
#define GDN_KERNEL_RECURRENCE 0 /* single-pass recurrence */
#define GDN_KERNEL_READOUT 1    /* O_t = Qf M_t (for a short call: with the state chain) */
#define GDN_KERNEL_GRAM 2       /* Gram pass: G_t, B_t per (head, frame) */
#define GDN_KERNEL_STATE 3      /* serial state pass over G_t, B_t */
#define GDN_KERNEL_BACKWARD 4   /* the backward's own kernels (its forward replay books as GRAM/STATE) */
#define GDN_KERNEL_TCONV 5      /* block-causal temporal convolution */
#define GDN_KERNEL_ATTN 6       /* block-causal softmax attention */
#define GDN_KERNEL_FUSED 7      /* one-launch forward (gram, state and readout roles in one kernel) */
#define GDN_KERNEL_SLOTS 8

typedef struct gdn_desc {
  int32_t abi_version; /* GDN_ABI_VERSION */
  int32_t B, H, T, S, D;
  int32_t io_dtype;    /* gdn_dtype */
  int32_t beta_mode;   /* gdn_beta_mode */
  uint32_t flags;      /* GDN_FLAG_* */
} gdn_desc;

/* ABI version the library was built with. */
int gdn_abi_version(void);

/* Static text for a status code (never NULL). */
const char* gdn_status_string(gdn_status s);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* gdn_last_error(void);

/*
 * Workspace bytes the library would like for `d` (all T frames staged at once,
 * capped at 1024 frames; the bf16 and e4m3 paths stage G_t, B_t and a bf16 state
 * snapshot per frame, between 2.5*D*D*2 and 3*D*D*2 bytes per head and frame); 0 if `d` is
 * invalid.  Any workspace of at
 * least gdn_workspace_min_size(d) bytes works: a smaller one makes the library
 * process the frames in more pieces, with bitwise the same results.
 */
size_t gdn_workspace_size(const gdn_desc* d);
size_t gdn_workspace_min_size(const gdn_desc* d);

/*
 * Host-only argument check shared by the two entry points; touches no device
 * and can run where there is no GPU.  `state_in_required` is 1 for
 * gdn_frame_step.  Returns GDN_OK or the first error found.
 */
gdn_status gdn_check_args(const gdn_desc* d, const void* q, const void* k, const void* v,
                          const float* gamma, const float* beta, const float* state_in,
                          const void* o, const float* state_out, const float* state_norms,
                          const void* workspace, size_t workspace_bytes,
                          int state_in_required);

/*
 * Whole-sequence forward (the offline / bidirectional-generation use of the
 * article's three single-GPU variants, and any call that owns all T frames).
 *   state_in     [B][H][D][D] or NULL for a zero initial state
 *   state_out    [B][H][D][D] or NULL (final state not needed)
 *   state_norms  [B][H][T] or NULL
 *   workspace    device scratch of workspace_bytes >= gdn_workspace_min_size(d)
 * Enqueues the work on `stream`; returns GDN_OK or an error status.
 */
gdn_status gdn_frame_forward(const gdn_desc* d, const void* q, const void* k, const void* v,
                             const float* gamma, const float* beta, const float* state_in,
                             void* o, float* state_out, float* state_norms,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_frame_forward for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid device allocation.  It
 * takes no workspace: it runs on a static device array of the library
 * (64 MiB, one copy on every GPU the library runs on, held until the process
 * ends), and calls nothing that allocates.  Same arguments, results (bitwise)
 * and stream behaviour as gdn_frame_forward, except: shapes whose workspace
 * would exceed the 64 MiB return GDN_ERR_WORKSPACE; GDN_FLAG_TIME_KERNELS
 * returns GDN_ERR_UNSUPPORTED; and the three-launch form, when it runs here,
 * stays on `stream` (no side stream).  All calls on one GPU share that GPU's
 * array, which keeps the last call's contents: calls that overlap on one GPU
 * (two streams, or two host threads) race and give undefined results; calls
 * in one stream's order do not.
 */
gdn_status gdn_frame_forward_noalloc(const gdn_desc* d, const void* q, const void* k, const void* v,
                                     const float* gamma, const float* beta, const float* state_in, void* o,
                                     float* state_out, float* state_norms, void* stream);

/*
 * One chunk of a chunk-causal streaming rollout (the article's chunk-causal
 * autoregressive variant; the cached-state hand-off of SANA-Video's block
 * KV cache): T = frames in this chunk (>= 1).  state_in is REQUIRED; state_out
 * may be NULL (read the cached state without committing it, e.g. for every
 * denoising step of a chunk) or equal to state_in (commit in place).
 * Running the frames of a sequence through consecutive gdn_frame_step calls,
 * the state handed from one to the next, gives bitwise the outputs and final
 * state of one gdn_frame_forward call over the whole sequence.
 */
gdn_status gdn_frame_step(const gdn_desc* d, const void* q, const void* k, const void* v,
                          const float* gamma, const float* beta, const float* state_in,
                          void* o, float* state_out, float* state_norms,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of gdn_frame_forward (bf16 I/O; the single-pass recurrence and e4m3
 * I/O have none): given dL/dO (d_out, [B][H][T][S][D] bf16) and optionally
 * dL/dM_final (d_state_out, fp32 [B][H][D][D]) for the forward over the same
 * q, k, v, gamma, beta and state_in, writes
 *   dq, dk, dv    [B][H][T][S][D] bf16   (each may be NULL: not computed)
 *   d_gamma, d_beta [B][H][T] fp32       (may be NULL)
 *   d_state_in    [B][H][D][D] fp32      (may be NULL)
 * The gradients are those of the recurrence in the SANA-WM news article
 * ("NVIDIA Apresenta SANA-WM ...", section "1. Atencao Linear Hibrida com Gated
 * DeltaNet (GDN)"), taken in exact arithmetic (ReLU's derivative is 0 at 0)
 * and evaluated with the same bf16 operands as the forward.  The forward is
 * replayed inside the call (its per-frame states are not kept by
 * gdn_frame_forward).  T <= 1024 frames per call; the workspace must hold
 * gdn_backward_workspace_size(d) bytes (0 if d is invalid or unsupported).
 * Longer sequences run in chunks, last chunk first: each chunk takes the
 * forward state at its start as state_in and the next chunk's d_state_in as
 * its d_state_out, which gives bitwise the gradients of one call.
 * Same conventions as gdn_frame_forward (device pointers, stream, errors);
 * no output may overlap an input or another output.
 */
size_t gdn_backward_workspace_size(const gdn_desc* d);
gdn_status gdn_frame_backward(const gdn_desc* d, const void* q, const void* k, const void* v,
                              const float* gamma, const float* beta, const float* state_in,
                              const void* d_out, const float* d_state_out,
                              void* dq, void* dk, void* dv, float* d_gamma, float* d_beta, float* d_state_in,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Training pair: a forward that keeps what the backward would otherwise replay,
 * and a backward that takes it.  gdn_frame_forward_train computes exactly what
 * gdn_frame_forward computes (bitwise the same o, state_out and state_norms)
 * and leaves, in `saved`, G_t = Kf^T Kf and B_t = Kf^T V_t of every frame and
 * bf16 snapshots of the initial state and of the state after every frame.
 * gdn_frame_backward_saved, given the same q, k, v, gamma, beta and that
 * saved buffer (unchanged), computes bitwise the gradients of
 * gdn_frame_backward (which replays the forward itself) without the replay.
 * bf16 I/O, the Gram pipeline, T <= 1024 frames per call.
 *   saved       device buffer of gdn_saved_size(d) bytes, 256-byte aligned,
 *               owned by the caller between the two calls (contents opaque)
 *   workspace   of the backward: gdn_backward_saved_workspace_size(d) bytes
 * Both sizes are 0 when d is invalid or not supported.  Other conventions as
 * for gdn_frame_forward and gdn_frame_backward.
 */
size_t gdn_saved_size(const gdn_desc* d);
size_t gdn_backward_saved_workspace_size(const gdn_desc* d);
gdn_status gdn_frame_forward_train(const gdn_desc* d, const void* q, const void* k, const void* v,
                                   const float* gamma, const float* beta, const float* state_in, void* o,
                                   float* state_out, float* state_norms, void* saved, size_t saved_bytes,
                                   void* stream);
gdn_status gdn_frame_backward_saved(const gdn_desc* d, const void* q, const void* k, const void* v,
                                    const float* gamma, const float* beta, const void* saved, size_t saved_bytes,
                                    const void* d_out, const float* d_state_out, void* dq, void* dk, void* dv,
                                    float* d_gamma, float* d_beta, float* d_state_in, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * Block-causal temporal convolution with a carried-token cache: the causal
 * FFN's temporal convolution in the talk "SANA-Video: Efficient Video
 * Generation with Block Linear Diffusion Transformer" (its closing part, the
 * two-block example: a zero token between blocks, the previous block's last
 * token carried in before the next block).  Depthwise, three taps along the
 * frame axis, at every spatial token and channel; for frame t of the call:
 *
 *   y[t]    = w[0]*left_t + w[1]*x[t] + w[2]*right_t + bias
 *   left_t  = x[t-1]; for t = 0 the cache (the previous call's last frame),
 *             zeros if cache_in is NULL
 *   right_t = x[t+1] when t+1 < T and t+1 starts no new block of `chunk`
 *             frames (blocks counted from the call's first frame), else zero
 *
 * chunk >= T is the two-sided convolution with zero padding (offline
 * generation); chunk = 1 is strictly causal.  Computed in fp32 with fused
 * multiply-adds in the order bias, left, current, right; y rounded to nearest
 * even.  cache_out (if not NULL) receives x[T-1], the carried token for the
 * next call: calls of one block each, the cache handed from one to the next,
 * give bitwise the y of one call over all frames.
 *
 * Layouts (device pointers): x, y [B][T][S][C] io_dtype (GDN_BF16 or GDN_F32);
 * w [3][C] fp32 (taps of the previous, current, next frame); bias [C] fp32 or
 * NULL; cache_in, cache_out [B][S][C] io_dtype or NULL.  C must be a multiple
 * of 8; x, y and the caches 16-byte aligned, w and bias 4-byte aligned.  y may
 * not overlap an input; cache_out may equal cache_in exactly (in-place cache
 * update) but not overlap it partially, nor overlap x, y, w or bias.  flags:
 * GDN_FLAG_TIME_KERNELS only.  Same stream and error conventions as the
 * calls above.
 */
typedef struct gdn_tconv_desc {
  int32_t abi_version; /* GDN_ABI_VERSION */
  int32_t B, T, S, C;
  int32_t chunk;       /* frames per block, >= 1 */
  int32_t io_dtype;    /* GDN_BF16 or GDN_F32 */
  uint32_t flags;
} gdn_tconv_desc;

gdn_status gdn_tconv_forward(const gdn_tconv_desc* d, const void* x, const float* w, const float* bias,
                             const void* cache_in, void* y, void* cache_out, void* stream);

/* Host-only argument check of gdn_tconv_forward (no device is touched). */
gdn_status gdn_tconv_check_args(const gdn_tconv_desc* d, const void* x, const float* w, const float* bias,
                                const void* cache_in, const void* y, const void* cache_out);

/*
 * Block-causal softmax attention: the periodic softmax attention blocks that
 * SANA-WM's hybrid keeps between its frame-wise GDN blocks (GeekNews summary
 * of SANA-WM, on the Hybrid Linear Diffusion Transformer; SANA-WM abstract).
 * Per (batch, head), with tokens frame-major (token i in frame i / S):
 *
 *   O = softmax(Q K^T * scale) V,  scale = desc.scale, or 1/sqrt(D) if 0
 *
 * masked block-causally over frames: the queries are the last Tq of the Tk
 * key frames, and a query in key frame f sees the keys of every frame before
 * the end of its block of `chunk` frames (blocks counted from key frame 0).
 * chunk >= Tk is full bidirectional attention; Tq < Tk is the streaming case
 * (queries of the current chunk against cached keys and values).
 *
 * Layouts (device pointers, bf16, 16-byte aligned): q, o [B][H][Tq][S][D];
 * k, v [B][H][Tk][S][D].  D in {16, 32, ..., 128}; one head's k (and v)
 * below 2 GiB (Tk*S*D*2 bytes).  fp32 accumulation and softmax (exp2 of scaled
 * scores, running max), the probabilities rounded to bf16 for the products
 * with V and with ones (the denominator), o rounded to nearest even.  o may not overlap q, k or v.  flags: GDN_FLAG_TIME_KERNELS only.
 * Same stream and error conventions as the calls above.
 */
typedef struct gdn_attn_desc {
  int32_t abi_version; /* GDN_ABI_VERSION */
  int32_t B, H, Tq, Tk, S, D;
  int32_t chunk;       /* frames per block, >= 1 */
  int32_t io_dtype;    /* GDN_BF16 */
  uint32_t flags;
  float scale;         /* softmax scale, finite and >= 0; 0 selects 1/sqrt(D) */
} gdn_attn_desc;

/*
 * workspace may be NULL.  With at least gdn_attention_workspace_size(d) bytes
 * (256-byte aligned, overlapping no tensor) the call may split each query
 * tile's keys over several workgroups and merge their partial softmax states
 * (fp32) in a second kernel: for launches with few query tiles, such as a
 * chunk of queries against a long cache.  The split changes the summation
 * order, so results differ from the unsplit call by rounding only; without a
 * workspace, queries of the last Tq frames give bitwise the rows of the
 * whole-sequence call.
 */
gdn_status gdn_attention_forward(const gdn_attn_desc* d, const void* q, const void* k, const void* v, void* o,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes for the key split gdn_attention_forward would choose on the
 * current device; 0 when the shape does not gain from it or d is invalid. */
size_t gdn_attention_workspace_size(const gdn_attn_desc* d);

/* Host-only argument check of gdn_attention_forward (no device is touched). */
gdn_status gdn_attention_check_args(const gdn_attn_desc* d, const void* q, const void* k, const void* v,
                                    const void* o, const void* workspace, size_t workspace_bytes);

/*
 * Device time of the kernels launched by calls that set GDN_FLAG_TIME_KERNELS
 * since the last reset: per kernel kind (GDN_KERNEL_*) the total milliseconds
 * and the number of launches.  Either pointer may be NULL.  Synchronises with
 * the recorded events.  `reset` != 0 clears the record after reading.
 * At most 65536 timed launches are kept unread; past that, timed calls launch
 * their kernels untimed until this call has read the record.
 * Returns GDN_OK or GDN_ERR_HIP.
 */
gdn_status gdn_kernel_times(double ms_out[GDN_KERNEL_SLOTS], int64_t launches_out[GDN_KERNEL_SLOTS],
                            int reset);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
