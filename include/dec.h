/*
 * dec.h -- C ABI of libdecmono.so: batch-1 (and small-batch) greedy decode of
 * a dense decoder-only transformer with fp16 weights on one AMD MI355X
 * (gfx950).
 *
 * What the library computes.  At batch size 1 each generated token is a
 * chain of matrix-vector products that reads every active weight once, so a
 * decode step is bound by memory bandwidth, not arithmetic
 * (hakusoku.com/story/7519, section GPU推論の速度制限要因：メモリ帯域幅).  The
 * whole step -- matrix products, attention, normalisation and sampling -- runs
 * as one resident GPU program with grid-wide phase barriers instead of one
 * kernel launch per operation (same page, sections
 * 標準推論スタックのボトルネックとKogの工夫 and
 * Kog Inference Engineの特徴とイノベーション).  Weights and the KV cache are
 * fp16 with no quantisation, pruning or cache compression (aether-echoes.com
 * operator view, section どう出したか).  The per-layer math (pre-norm RMSNorm,
 * rotary embedding on adjacent pairs, multi-head attention, SwiGLU MLP,
 * untied LM head, greedy argmax with the lowest index winning ties) is fixed
 * by the model description below.
 *
 * Provenance of the calls.  The pages describe a system, not a programming
 * interface: they name no API.  The calls below are this library's contract
 * for the decode path (a handle made from a model description and weights;
 * prefill; one step yielding a token and optionally its logits; reset), and
 * each call's comment names the passage whose operation it carries out.
 * Calls that only serve tests or measurement say so.
 *
 * Conventions
 *  - Every function returns a dec_status (0 = OK, negative = error) unless
 *    stated; on error dec_last_error() describes it.
 *  - Pointers named host_* or out_* and token/logit arrays are HOST memory.
 *    The library never retains caller pointers past the call, except the
 *    optional device arena and stream passed to dec_init.
 *  - A handle is not thread-safe; distinct handles are independent.
 *  - All calls that run GPU work are synchronous with respect to the handle's
 *    stream unless stated (dec_step with out_tok == NULL and out_logits ==
 *    NULL is asynchronous; its input arrays are still read during the call
 *    only).
 */
#ifndef DECMONO_DEC_H
#define DECMONO_DEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DEC_ABI_VERSION 2

typedef enum dec_status {
  DEC_OK = 0,
  DEC_ERR_INVALID_ARG = -1,   /* NULL handle/pointer, negative count, ...          */
  DEC_ERR_BAD_DESC = -2,      /* model description violates the rules below         */
  DEC_ERR_WEIGHTS = -3,       /* weight file or tensor list missing/short/mismatched */
  DEC_ERR_NO_DEVICE = -4,     /* no usable gfx950 device                             */
  DEC_ERR_OOM = -5,           /* device or pinned-host allocation failed / arena small */
  DEC_ERR_CONTEXT_FULL = -6,  /* position would pass max_ctx                         */
  DEC_ERR_STATE = -7,         /* call not valid in the handle's state                */
  DEC_ERR_TOKEN_RANGE = -8,   /* token id outside [0, vocab)                         */
  DEC_ERR_DEVICE = -9,        /* a HIP runtime call failed                           */
  DEC_ERR_TIMEOUT = -10,      /* an in-kernel barrier wait passed the watchdog bound */
  DEC_ERR_UNSUPPORTED = -11   /* valid request this library does not implement       */
} dec_status;

/*
 * Model description.  Rules (DEC_ERR_BAD_DESC otherwise):
 *   n_layers >= 1; d_model >= 8, a multiple of 8 and even;
 *   n_kv_heads == n_heads >= 1 (multi-head attention);
 *   head_dim in {8, 16, 32, 64, 128};
 *   n_heads*head_dim may differ from d_model and must be a multiple of 8;
 *   d_ffn >= 8, a multiple of 8;
 *   1 <= lm_vocab <= vocab, lm_vocab even;
 *   1 <= max_ctx <= 65536; batch >= 1; rms_eps > 0; rope_base > 1;
 *   flags: 0, DEC_FLAG_BATCHED_PREFILL or DEC_FLAG_MATRIX_PREFILL (batch 1
 *   only; not both).
 * Limits of this library (DEC_ERR_UNSUPPORTED): d_model, n_heads*head_dim and
 * d_ffn <= 8192; batch <= 8; with batch > 1, d_model <= 2560 and d_ffn,
 * n_heads*head_dim <= 7680 after rounding up to a multiple of 512 (every
 * sequence's matrix-product input is held on chip, in fp16).
 * Shapes of the weight tensors follow from it (see dec_weights_src).
 *
 * Mixture of experts (n_experts > 0).  Every layer's MLP is then n_experts
 * SwiGLU experts of width d_ffn whose matrices are FP8 E4M3 codes with one
 * float32 scale per output row; a bias-free fp16 router [n_experts, d_model]
 * applied to the same normed vector picks the top_k experts with the largest
 * logits (the lower expert index first on equal logits), and their outputs
 * are added with the softmax of those top_k logits as weights.  This is the
 * pages' next milestone, large mixture-of-experts models read at their
 * active-parameter size with FP8 expert weights (page
 * 標準GPUによるリアルタイムLLM推論, section Hackerたちの意見; page
 * 「ソフトウェア・ファースト」戦略でGPUの限界を突破…, section
 * 今後のマイルストーンと課題).  Rules (DEC_ERR_BAD_DESC otherwise):
 * n_experts == 0 and top_k == 0 for a dense model; else 2 <= n_experts <= 64,
 * n_experts even, 1 <= top_k <= min(n_experts, 8).  Limits
 * (DEC_ERR_UNSUPPORTED): batch 1, flags 0 or DEC_FLAG_EXPERTS_MXFP4, d_model
 * and d_ffn multiples of 16 (32 with MXFP4), top_k * d_ffn <= 7168, each layer's expert matrices under 2 GiB of
 * codes; weights from host tensors only (not a DECW file), not with
 * dec_init_noalloc, dec_pack or DEC_DEBUG_MULTILAUNCH.  Numerics: the
 * router's top_k choice is made on fp32 logits; a choice between two
 * experts whose logits differ by less than the accumulated rounding can
 * differ from an exact evaluation's (see dec_read_routes).
 *
 * Batch.  batch > 1 decodes that many independent sequences in lockstep (same
 * position, one pass over the weights per step serves all of them); each has
 * its own KV cache.  Sequence b's tokens and logits are the ones it would get
 * alone, up to rounding: the batched kernel rounds each matrix product's input
 * vector (x*g, the attention output, the SwiGLU output) to fp16, where the
 * batch-1 kernel keeps it in fp32.
 */
/*
 * DEC_FLAG_BATCHED_PREFILL: dec_prefill runs the prompt 8 positions at a time
 * through the batched (matrix-core) kernel instead of one position per step
 * of the decode kernel.  The handle keeps a second, tiled copy of the
 * weights (see dec_pack) and its per-position buffers hold 8 columns; the
 * shape limits of batch > 1 apply.  Numerics: each matrix product's input is
 * rounded to fp16 as in the batched kernel, so the prompt's cache entries and
 * logits differ from the default prefill's by that rounding.  Decode steps
 * are unchanged.
 */
#define DEC_FLAG_BATCHED_PREFILL 0x2u
/*
 * DEC_FLAG_MATRIX_PREFILL: dec_prefill runs all prompt positions through
 * each weight matrix at once, as matrix products on the matrix cores (up to
 * 2048 positions per pass over the weights), with a tiled causal attention
 * over the cache; the time to first token is one of the speed figures of
 * hakusoku.com/story/7519, section 単一リクエストLLMデコード速度の重要性.
 * Needs head_dim >= 32 and d_model, n_heads*head_dim, d_ffn multiples of 32
 * (DEC_ERR_UNSUPPORTED otherwise).  The handle's arena holds a workspace of
 * about min(max_ctx, 2048) x (4 d_model + 2 max(d_model, H hd) + 2 H hd +
 * 2 d_ffn + 4) bytes plus up to 32 MB of partial sums (dec_arena_bytes
 * includes it).  Numerics: the products' inputs are rounded
 * to fp16 as with DEC_FLAG_BATCHED_PREFILL, and so are the rotated queries and
 * the softmax weights of the attention products.  Decode steps are unchanged.
 */
#define DEC_FLAG_MATRIX_PREFILL 0x4u
/*
 * DEC_FLAG_EXPERTS_MXFP4 (mixture of experts only): the expert matrices are
 * OCP microscaling MXFP4 blocks instead of E4M3 codes with row scales --
 * FP4 E2M1 codes two to a byte (element 2i in the low nibble) and one E8M0
 * scale, 2^(s - 127), per 32 consecutive weights of a row: the pages' FP4
 * expert format (page 標準GPUによるリアルタイムLLM推論, section Hackerたちの意見).
 * Needs d_model and d_ffn multiples of 32.  Tensors (see dec_weights_src):
 * Wg8, Wu8 [E*F, d/2] and Wd8 [E*d, F/2] uint8 code pairs; sg, su
 * [E*F, d/32] and sd [E*d, F/32] uint8 scales.
 */
#define DEC_FLAG_EXPERTS_MXFP4 0x8u

typedef struct dec_model_desc {
  int32_t n_layers;
  int32_t d_model;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t d_ffn;
  int32_t vocab;      /* rows of the embedding table                  */
  int32_t lm_vocab;   /* rows of the LM head (a vocabulary shard if < vocab) */
  int32_t max_ctx;    /* KV-cache positions per sequence               */
  int32_t batch;      /* sequences decoded together                    */
  float rms_eps;
  float rope_base;
  uint32_t flags;     /* 0, DEC_FLAG_BATCHED_PREFILL, DEC_FLAG_MATRIX_PREFILL or (experts) DEC_FLAG_EXPERTS_MXFP4 */
  int32_t n_experts;  /* 0: dense MLP; else experts per layer (mixture of experts) */
  int32_t top_k;      /* experts each token uses (mixture of experts), else 0 */
} dec_model_desc;

/*
 * Weight source: exactly one of `path` or `host_tensors` is non-NULL.
 *
 * host_tensors: n_tensors pointers to fp16 bit patterns (IEEE binary16,
 * little-endian), matrices [out, in] row-major, in canonical order
 *   E [vocab, d]
 *   for each layer: g_attn [d], Wq [H*hd, d], Wk [H*hd, d], Wv [H*hd, d],
 *                   Wo [d, H*hd], g_ffn [d], Wg [F, d], Wu [F, d], Wd [d, F]
 *   g_final [d], W_lm [lm_vocab, d]
 * so n_tensors == 1 + 9*n_layers + 2.  The caller owns the buffers; they are
 * read during dec_init only.
 *
 * Mixture of experts (n_experts = E > 0, expert width F = d_ffn): the layer's
 * Wg, Wu, Wd are replaced by seven tensors, so n_tensors == 1 + 13*n_layers
 * + 2, and each pointer's bytes are read as the tensor's own element type:
 *   for each layer: g_attn, Wq, Wk, Wv, Wo, g_ffn (fp16 as above),
 *                   Wr  [E, d]      fp16 router,
 *                   Wg8 [E*F, d]    uint8 E4M3 codes,  sg [E*F] float32 row scales,
 *                   Wu8 [E*F, d]    uint8 E4M3 codes,  su [E*F] float32,
 *                   Wd8 [E*d, F]    uint8 E4M3 codes,  sd [E*d] float32
 * Expert e owns rows e*F .. e*F+F-1 of Wg8/Wu8 (and of sg/su) and rows
 * e*d .. e*d+d-1 of Wd8 (and of sd); its matrix element is
 * value(code) * scale of the element's row.
 *
 * path: a DECW weight file (format below).  Its description must equal the
 * one passed to dec_init in every shape field.
 *
 * DECW file, little-endian:
 *   0   char[4]  "DECW"
 *   4   uint32   version (1)
 *   8   uint32   n_tensors
 *   12  uint32   reserved (0)
 *   16  int32[10] n_layers d_model n_heads n_kv_heads head_dim d_ffn vocab
 *                lm_vocab max_ctx batch; float32 rms_eps, rope_base;
 *                uint32 flags; 4 bytes padding   (56 bytes, ends at 72)
 *   72  n_tensors entries of 40 bytes:
 *         uint32 index (== position in the canonical order)
 *         uint32 dtype (1 = fp16)
 *         uint32 ndim (1 or 2), uint32 reserved
 *         uint32 dim0, uint32 dim1 (dim1 = 1 when ndim == 1)
 *         uint64 offset (from file start, multiple of 256)
 *         uint64 nbytes (== 2*dim0*dim1)
 *   payload: each tensor at its offset, row-major fp16.
 */
typedef struct dec_weights_src {
  const char* path;
  const uint16_t* const* host_tensors;
  int32_t n_tensors;
} dec_weights_src;

/* debug_flags */
#define DEC_DEBUG_MULTILAUNCH 0x1u  /* one kernel launch per phase instead of one
                                       resident kernel with grid barriers (the
                                       "one launch per op" stack, for comparison) */
#define DEC_DEBUG_TRACE 0x2u        /* record per-phase wall-clock stamps (see
                                       dec_read_trace) */
#define DEC_DEBUG_FENCED 0x4u       /* also issue agent-scope release and acquire
                                       fences around every grid barrier; results
                                       are bitwise those of the default path */
#define DEC_DEBUG_STRESS 0x8u       /* barrier stress: each workgroup waits a
                                       pseudo-random 0-2 us before every arrival,
                                       and every exchange buffer is filled with
                                       NaN between its last read and its next
                                       write; results are bitwise those of the
                                       default path unless a read races a write.
                                       Not with DEC_DEBUG_MULTILAUNCH. */

/*
 * Init options (NULL = all defaults).
 *   device:      HIP device ordinal.
 *   stream:      hipStream_t to run on (e.g. torch.cuda.Stream().cuda_stream);
 *                NULL: the library creates and owns a stream.  A caller stream
 *                must outlive the handle.
 *   arena, arena_bytes: optional caller-owned device memory that holds every
 *                device buffer of the handle (weights, KV cache, activations,
 *                barrier words); must be 256-byte aligned, at least
 *                dec_arena_bytes() long and outlive the handle.  NULL: the
 *                library allocates with hipMalloc.
 *   debug_flags: DEC_DEBUG_*.
 *   watchdog_us: bound on every in-kernel barrier wait; on expiry the kernel
 *                exits and the call returns DEC_ERR_TIMEOUT.  0 = 2,000,000.
 *   grid:        workgroups of the resident kernel; 0 = one per compute unit.
 *                It must be at least batch x n_heads (8 x n_heads with
 *                DEC_FLAG_BATCHED_PREFILL), else DEC_ERR_UNSUPPORTED.
 *   serve_idle_us: 0 = every dec_step is a kernel launch of its own.  1 ..
 *                10,000,000 = decode server: one resident launch serves a
 *                run of dec_step calls, which post their steps to it through
 *                host-pinned memory (allocated with the handle) instead of
 *                launching; the launch ends when any other call on the
 *                handle needs the stream (dec_sync, dec_generate,
 *                dec_prefill, dec_reset, dec_read_kv, dec_read_trace,
 *                dec_free), or by itself after serve_idle_us without a step
 *                (the next dec_step then starts a new one).  While it runs it
 *                holds every compute unit of the device: other work on the
 *                handle's stream, and work on other streams that needs a
 *                compute unit, waits for its end, so call dec_sync before
 *                such work.  Not with dec_init_noalloc or
 *                DEC_DEBUG_MULTILAUNCH (DEC_ERR_INVALID_ARG).
 *                The pages' GPU-resident program that removes kernel
 *                boundaries and host scheduling between tokens (page
 *                標準GPUによるリアルタイムLLM推論, section
 *                標準推論スタックのボトルネックとKogの工夫).
 */
typedef struct dec_init_opts {
  int32_t device;
  int32_t grid;
  void* stream;
  void* arena;
  size_t arena_bytes;
  uint32_t debug_flags;
  int32_t watchdog_us;
  int32_t serve_idle_us;
  int32_t reserved[5];
} dec_init_opts;

typedef struct dec_handle dec_handle;

/* ABI version of the loaded library (DEC_ABI_VERSION it was built with).
 * Library bookkeeping; no passage of the pages. */
int32_t dec_abi_version(void);

/*
 * Bytes of device memory a handle for `desc` needs (weights, KV cache,
 * activations and control words), for a caller-provided arena.  Host only;
 * needs no GPU.  grid = workgroups the kernel will use (0 = 256).
 * Memory planning for the weights and the KV cache the bandwidth bound counts
 * (page 標準GPUによるリアルタイムLLM推論, section
 * GPU推論の速度制限要因：メモリ帯域幅).
 */
int dec_arena_bytes(const dec_model_desc* desc, int32_t grid, size_t* out_bytes);

/*
 * Validate `desc` without touching any device.  DEC_OK or DEC_ERR_BAD_DESC /
 * DEC_ERR_UNSUPPORTED with the reason in dec_last_error(NULL).  The shape
 * rules are this library's (the pages give only a 2B-class, 25-layer, fp16
 * model with a 4096-token context: aether-echoes operator view, section
 * どう出したか).
 */
int dec_check_desc(const dec_model_desc* desc);

/*
 * Read and validate the header and tensor table of a DECW file against the
 * rules above (magic, version, count, dtypes, shapes, offsets, file size).
 * Fills *out_desc from the header.  Host only.  DEC_ERR_WEIGHTS on any defect.
 * The pages define no weight file; DECW is this library's inference-only
 * format for fp16 weights with no quantisation (studioglobal.ai article,
 * section Laneformer 2B: 実証済みの性能).
 */
int dec_weights_file_check(const char* path, dec_model_desc* out_desc);

/*
 * Create a handle: validate, read/pack the weights on the host, upload them,
 * allocate the KV cache for batch x max_ctx positions and build the rotary
 * table (cos/sin of p * rope_base^(-2i/head_dim), computed in double on the
 * host, stored as fp32).  Position starts at 0.  On failure *out is NULL and
 * dec_last_error(NULL) holds the reason.  The weights are packed once into
 * the layout the decode kernel streams, the hand-controlled low-level layout
 * and execution the pages credit for reaching bandwidth speed (page
 * 標準GPUによるリアルタイムLLM推論, section Kog Inference Engineの特徴とイノベーション).
 */
int dec_init(const dec_model_desc* desc, const dec_weights_src* weights,
             const dec_init_opts* opts, dec_handle** out);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Creates the
 * same handle as dec_init, and every other call works on it unchanged, but:
 *   - opts, opts->arena and opts->stream are required (else
 *     DEC_ERR_INVALID_ARG).  The arena holds the weights, gains, rotary table
 *     and KV cache; an arena of dec_arena_bytes() bytes is always large
 *     enough, and only its leading part is used;
 *   - the kernels' scratch -- residual stream and the other exchange vectors,
 *     attention and argmax partials, logits, token buffers, barrier counters,
 *     the device copies of the parameter block and (DEC_DEBUG_TRACE) the
 *     trace -- lives in a fixed array inside the library,
 *     DEC_NOALLOC_SCRATCH_BYTES per device, which that device holds until the
 *     process exits.  A description whose scratch is larger is rejected with
 *     DEC_ERR_UNSUPPORTED (the 2.3B shape needs about 1 MiB at batch 1 and
 *     4 MiB at batch 8; the trace adds 8 MiB at 256 workgroups).
 * Neither this call nor any later call on the handle allocates device memory
 * (no hipMalloc, hipFree or allocating library routine).  Init clears the
 * part of the array it uses: a previous user's contents are never read.  A
 * device has one array, so one no-allocation handle at a time may use it:
 * while one is alive, dec_init_noalloc on the same device returns
 * DEC_ERR_STATE (two handles would race on the shared array); dec_free
 * releases it.  Other errors as dec_init.
 */
#define DEC_NOALLOC_SCRATCH_BYTES (16u << 20)
int dec_init_noalloc(const dec_model_desc* desc, const dec_weights_src* weights,
                     const dec_init_opts* opts, dec_handle** out);

/*
 * Prefill: requires position 0 (fresh or after dec_reset), else
 * DEC_ERR_STATE.  tokens: host int32 [batch * n] (sequence-major), 1 <= n <=
 * max_ctx.  Runs positions 0..n-1 (keys/values of every position enter the
 * cache) and returns the greedy next token of each sequence in out_tok
 * [batch] (host, required) and, if out_logits != NULL, the last position's
 * logits [batch * lm_vocab] (host, fp32).  Position becomes n.
 * The prompt phase before decoding; its duration is the time to first token,
 * one of the three speed axes the pages name (page 標準GPUによるリアルタイム
 * LLM推論, section 単一リクエストLLMデコード速度の重要性).
 */
int dec_prefill(dec_handle* h, const int32_t* tokens, int32_t n,
                int32_t* out_tok, float* out_logits);

/*
 * One decode step at the current position p.  Input token: force_tok[batch]
 * (host) if non-NULL (teacher forcing), else the previous greedy output kept
 * on the device.  force_tok is read during the call only: its values travel
 * in the kernel launch's arguments.  Appends the keys/values of position p,
 * advances to p+1 and produces the greedy token.  out_tok [batch] (host) and
 * out_logits [batch * lm_vocab] (host) are optional; with both NULL the call
 * only enqueues work on the stream and returns without waiting (use dec_sync;
 * a device error such as DEC_ERR_TIMEOUT then surfaces at the next
 * synchronous call).  On a decode-server handle (serve_idle_us > 0) the step
 * is posted to the running server launch (started if none runs); with both
 * outputs NULL the call returns once it is posted, waiting only while 64
 * posted steps are unfinished.  DEC_ERR_CONTEXT_FULL if p == max_ctx; DEC_ERR_STATE
 * before any prefill; DEC_ERR_TOKEN_RANGE for a forced token outside
 * [0, vocab).
 * One step is one pass over every active weight plus the KV cache read, the
 * quantity the bandwidth bound prices (page 標準GPUによるリアルタイムLLM推論,
 * section GPU推論の速度制限要因：メモリ帯域幅), with matrix products,
 * attention, normalisation and sampling in one resident program (same page,
 * section Kog Inference Engineの特徴とイノベーション); sampling is greedy
 * (studioglobal.ai article, table under Laneformer 2B: 実証済みの性能).
 */
int dec_step(dec_handle* h, const int32_t* force_tok, int32_t* out_tok, float* out_logits);

/*
 * n_steps greedy steps inside one kernel launch, each step fed the previous
 * step's token on the device.  Same result as n_steps dec_step calls with
 * force_tok == NULL.  out_toks: host int32 [n_steps * batch] (step-major).
 * One GPU-resident program for many tokens, without a kernel boundary or host
 * scheduling between them (page 標準GPUによるリアルタイムLLM推論, section
 * 標準推論スタックのボトルネックとKogの工夫).
 */
int dec_generate(dec_handle* h, int32_t n_steps, int32_t* out_toks);

/* Wait for all work enqueued on the handle's stream; reports deferred errors.
 * Library bookkeeping; no passage of the pages. */
int dec_sync(dec_handle* h);

/* Position -> 0.  The cache is logically empty (overwritten, not cleared).
 * Starts a new request on the same weights (the pages' single-request
 * serving, section 単一リクエストLLMデコード速度の重要性). */
int dec_reset(dec_handle* h);

/* Current position (number of cached positions), or -1 for a NULL handle.
 * Library bookkeeping; no passage of the pages. */
int32_t dec_position(const dec_handle* h);

/*
 * Copy cached keys and values of positions [0, n_pos) of one layer and one
 * sequence to host memory as fp16 bits, each [n_heads, n_pos, head_dim].
 * Either output may be NULL.  For tests and inspection; synchronous.  The
 * cache is the KV term of the bandwidth bound (page 標準GPUによるリアルタイム
 * LLM推論, section GPU推論の速度制限要因：メモリ帯域幅).
 */
int dec_read_kv(dec_handle* h, int32_t layer, int32_t seq, int32_t n_pos,
                uint16_t* host_k, uint16_t* host_v);

/*
 * Mixture-of-experts models: the experts the router chose at positions
 * [pos0, pos0 + n_pos), copied to host as int32 [n_pos][n_layers][top_k]
 * (largest logit first).  Every step and prefill records its positions'
 * choices; a position not yet computed reads as -1.  DEC_ERR_STATE for a
 * dense model.  For tests and inspection (a choice between experts whose
 * logits nearly tie can legitimately differ from an exact evaluation's);
 * synchronous.  The routing the pages' mixture-of-experts projection
 * assumes (page 標準GPUによるリアルタイムLLM推論, section Hackerたちの意見).
 */
int dec_read_routes(dec_handle* h, int32_t pos0, int32_t n_pos, int32_t* out_routes);

/*
 * Phase trace of the most recent launch (handle created with DEC_DEBUG_TRACE).
 * For each workgroup g the kernel stores, in order, the device wall-clock
 * time at the start and at the end of every phase it ran: stamps
 * [g*stride + 2j] and [g*stride + 2j + 1] for the launch's j-th phase
 * (stamps beyond `stride` are dropped).  *out_grid and *out_stride receive
 * the grid and the stride; *out_hz the clock rate.  host: uint64
 * [grid*stride] or NULL to query the sizes only.  Synchronous.
 * Measurement aid for finding where the microseconds of a step go (page
 * 標準GPUによるリアルタイムLLM推論, section Kog Inference Engineの特徴とイノベーション).
 */
int dec_read_trace(dec_handle* h, uint64_t* host, int32_t* out_grid, int32_t* out_stride, double* out_hz);

/* Release every resource of the handle (not a caller arena or stream).
 * Library bookkeeping; no passage of the pages. */
void dec_free(dec_handle* h);

/*
 * Measurement aid: the sustained HBM read rate of a plain stream on this
 * device, the ceiling the decode kernel's weight stream is compared with
 * (the bandwidth bound of page *標準GPUによるリアルタイムLLM推論：リクエストあ
 * たり3,000トークン/秒*, section *GPU推論の速度制限要因：メモリ帯域幅*, prices
 * every byte at the device's bandwidth).  One 512-thread workgroup per
 * compute unit; each wave reads its own contiguous share of the buffer's
 * 1 KB blocks with 16-byte non-temporal loads, eight blocks in flight (the
 * access pattern of the decode kernel's weight streams).
 *   device:   HIP device ordinal.
 *   bytes:    buffer size, at least 64 MiB and at most 64 GiB; rounded down
 *             to a multiple of 1 MiB.  Allocated on the device, filled, read
 *             once untimed, then `reps` times timed with HIP events, freed.
 *   reps:     1..100.
 *   out_gbps: bytes * reps / elapsed / 1e9.
 * Synchronous.  Returns DEC_ERR_INVALID_ARG for bad arguments, DEC_ERR_OOM if
 * the buffer cannot be allocated, DEC_ERR_DEVICE for another HIP error.  It
 * shares the device with any running decode work, so call it when none runs.
 */
int dec_stream_ceiling(int32_t device, uint64_t bytes, int32_t reps, double* out_gbps);

/*
 * Last error text of the handle, or of the calling thread's last failed
 * handle-less call (dec_init, dec_check_desc, ...) when h == NULL.  Never NULL.
 * Library bookkeeping; no passage of the pages.
 */
const char* dec_last_error(const dec_handle* h);

/*
 * Host packer, exposed for inspection and tests (no GPU needed).
 * dec_packed_bytes: size of the packed fp16 weight image for desc.
 * dec_pack: write that image to host memory dst (dst_bytes >= the size) from
 * the canonical tensor list (see dec_weights_src).  Layout of the image, in
 * fp16 elements, each region 128-element aligned:
 *   for each layer l:
 *     Wqkv[l]  [3*H*hd, d]   rows: Wq rows, then Wk rows, then Wv rows
 *     Wo[l]    [d, H*hd]
 *     Wgu[l]   [2*F, d]      row 2f = Wg row f, row 2f+1 = Wu row f
 *     Wd[l]    [d, F]
 *   E        [vocab, d]
 *   W_lm     [lm_vocab, d]
 * Gains are not part of the image (they are uploaded as fp32).
 * With batch == 1 every matrix is row-major.  With batch > 1 every matrix
 * except E is stored in tiles of 16 rows x 32 columns (the A operand of the
 * matrix-core instruction the batched kernel uses): tile (g, j) covers rows
 * 16g..16g+15 and columns 32j..32j+31, tiles follow each other row-group
 * first (index g * ceil(cols/32) + j), and inside a tile the 8 elements at
 * element offset 8*l are row 16g + l%16, columns 32j + 8*(l/16) .. +7, for
 * l = 0..63.  Rows and columns past the matrix are zero; each matrix region
 * is ceil(rows/16) * ceil(cols/32) * 512 elements.
 * The weight pre-pack into the layout the kernel streams (page
 * 標準GPUによるリアルタイムLLM推論, section Kog Inference Engineの特徴とイノベーション).
 */
int dec_packed_bytes(const dec_model_desc* desc, size_t* out_bytes);
int dec_pack(const dec_model_desc* desc, const uint16_t* const* host_tensors,
             int32_t n_tensors, void* dst, size_t dst_bytes);

#ifdef __cplusplus
}
#endif
#endif /* DECMONO_DEC_H */
