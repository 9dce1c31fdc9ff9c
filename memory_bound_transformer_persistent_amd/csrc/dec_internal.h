// Internal definitions shared by the host runtime (dec_host.cpp) and the
// device code (dec_kernels.hip, dec_matrix.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP__)
#define DEC_HD __host__ __device__
#else
#define DEC_HD
#endif

namespace decmono {

constexpr int kThreads = 512;               // threads per workgroup (8 wave64)
constexpr int kWaves = kThreads / 64;
constexpr int kGroups = 63;                 // barrier groups: workgroup b is in group b % 63 (lane 63 of the poll reads the error word)
constexpr int kMaxK = 8192;                 // longest GEMV row supported (16 pieces per lane)
constexpr int kChunkMin = 32;               // shortest attention chunk (positions)
constexpr int kChunkMax = 2048;
constexpr int kTraceStride = 4096;          // trace stamps kept per workgroup per launch
constexpr int kOutFloats = 2048;            // LDS: one phase's GEMV results of a workgroup
constexpr int kOwnFloats = 256;             // LDS: a workgroup's rows of the residual stream (all sequences)
// Batched decode (up to kMaxBatch sequences at the same position): the GEMV
// inputs of every sequence sit in LDS as fp16, side by side, so one pass over
// the weights serves all of them.  Limits that keep them in LDS:
constexpr int kMaxBatch = 8;
// mixture of experts: limits, the kernel-kind value of the batch-1
// mixture-of-experts kernel, and where a workgroup's gate/up results start
// in its LDS result buffer (the router's logits come first)
constexpr int kMoeMaxExperts = 64;
constexpr int kMoeMaxTopK = 8;
constexpr int kMoeKernel = 0;
constexpr int kMoeOutPairs = 64;
constexpr int kMoeScaleFloats = 512;   // LDS for the down phase's row scales of every chosen expert
constexpr int kMoeWrElems = 768;       // LDS fp16 elements for the router's columns of a workgroup's residual rows
constexpr int kBatchSpanD = 2560;           // padded d_model (input of QKV, GU, LM; staged in fp32 too)
constexpr int kBatchSpanK = 7680;           // padded d_ffn and n_heads*head_dim
// The batched kernel multiplies weights by the inputs with MFMA
// (v_mfma_f32_16x16x32_f16): its weights are packed in 1 KB tiles of 16 rows
// x 32 columns, and a workgroup owns whole 16-row groups of every matrix.
constexpr int kTileRows = 16;
constexpr int kTileCols = 32;
constexpr int kTileElems = kTileRows * kTileCols;
constexpr int kLdsBytes = 160 * 1024;       // dynamic LDS per workgroup; > half a CU's 160 KB,
                                            // so exactly one workgroup runs per compute unit

// The no-allocation handle (dec_init_noalloc) keeps its scratch -- everything
// in the arena from the residual stream on: exchange vectors, partials,
// logits, token buffers, control words, parameter blocks, trace -- in a
// fixed device array of this size, one per device.
constexpr size_t kNoallocScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;

// Control words (uint32 index into Params::ctl); each on its own 256-byte line.
constexpr int kCtlGlobal = 0;               // arrivals of group leaders (cumulative)
constexpr int kCtlGroup0 = 64;              // group k counter at kCtlGroup0 + 64*k
constexpr int kCtlErr = 64 * (1 + kGroups); // first error code raised by any workgroup
constexpr int kCtlHead0 = 64 * (2 + kGroups);  // per-head arrival counters of attention chunks
constexpr int kMaxHeads = 1024;
constexpr int kCtlWords = kCtlHead0 + kMaxHeads;

// Phases of one token.  Per layer: QKV, ATTN, O, GU, DOWN; then LM and ARGMAX
// when the token's logits are wanted.
enum Phase : int { PH_QKV = 0, PH_ATTN = 1, PH_O = 2, PH_GU = 3, PH_DOWN = 4, PH_LM = 5 };
constexpr int kPhasesPerLayer = 5;

enum TokSrc : int { TOK_PROMPT = 0, TOK_DEVICE = 1 };

// Error codes raised on the device (same values as dec_status).
constexpr int kDevErrTimeout = -10;

// Decode server: one resident launch serves a run of dec_step calls.  The
// host posts step k of the launch as request k in a mailbox in host-pinned,
// coherent memory that the device reads through its own mapping.  Only
// workgroup 0 reads the mailbox; it copies each request into device slots
// (kSrvCopies replicas, so polling workgroups spread over memory channels)
// that the other workgroups read.  `ctl` holds the number of requests posted
// to the running launch, plus kMailClosed once no request follows: the host
// sets it to end the launch, and workgroup 0 sets it when no request came for
// the idle bound.  Both post and close with a compare-and-swap on `ctl`, so a
// request is either posted before the close or refused by it, for host and
// device alike.
constexpr int kMailRing = 64;          // requests in flight at most
constexpr int kReqWords = 16;          // per request: flags, then the batch's input tokens
constexpr int kReqForce = 1;           // request flag: the step's input tokens are given
constexpr int kReqLogits = 2;          // request flag: store the step's logits for the host
constexpr uint32_t kMailClosed = 0x80000000u;
constexpr int kSrvCopies = 8;
struct Mailbox {
  uint32_t ctl;                        // requests posted | kMailClosed
  uint32_t pad0[63];
  uint32_t done;                       // requests completed (their tokens are in tok)
  uint32_t pad1[63];
  int32_t req[kMailRing][kReqWords];   // request k in slot k % kMailRing
  int32_t tok[kMailRing][kMaxBatch];   // greedy tokens of completed request k
};
// device slot of request k (words): [0,1] tag, [2] flags, [3 ..] tokens; the
// tag is (launch epoch << 32) | (k + 1), with kMailClosed when the launch ends at k
constexpr int kSrvSlotWords = kSrvCopies * kMailRing * kReqWords;

struct Params {
  int L, d, H, hd, F, V, Vlm, max_ctx, q;   // q = H*hd
  float eps;
  const uint16_t* w;          // packed weight image (fp16 bits)
  size_t layer_stride;        // elements between consecutive layers in the image
  size_t off_qkv, off_o, off_gu, off_d;   // element offsets inside a layer
  size_t off_E, off_lm;       // element offsets of the embedding and the LM head
  const float* gains;         // [L][2][d] (attn, ffn) then g_final [d]
  const float* rope;          // [max_ctx][hd/2][2] (cos, sin)
  int B;                      // columns of the batched kernel: sequences decoded together (batch)
  int cols_pos;               // 1: the columns are consecutive positions of one sequence (batched prefill)
  uint16_t* kv;               // [L][2][B][H][max_ctx][hd] fp16 (one sequence when cols_pos)
  float* x;                   // residual stream [B][d] (the batched kernel keeps its rows in LDS and stores them here only where a launch ends)
  float* qkv;                 // [B][3q]: rotated, scaled q in the first q of each sequence
  float* att_o;               // attention output [B][q] (batch 1, fp32)
  uint16_t* att_o16;          // attention output [B][q] (batch > 1, fp16; same memory as att_o)
  float* part;                // attention partial sums [B*H][max_chunks][hd]
  float* pml;                 // attention partial (max, sum) [B*H][max_chunks][2]
  float* act;                 // SwiGLU output [F] (batch 1, fp32)
  uint16_t* act16;            // SwiGLU output (batch > 1, fp16 in 8-row blocks, see blk8; same memory as act)
  float* logits;              // [B][Vlm]
  float* amax_v;              // per-workgroup best logit: [G] at batch 1, [G][kMaxBatch] batched
  int* amax_i;                // its row (lowest on ties), same layout
  int* tok_cur;               // token each sequence's next step consumes [B]
  int* tok_out;               // greedy tokens of a launch [max_ctx][B]
  const int* prompt;          // tokens of a prompt launch [B][n_tok]
  uint32_t* ctl;              // control words
  int max_chunks;
  uint32_t watchdog_ticks;    // bound on one barrier wait, in wall-clock ticks
  uint64_t* trace;            // optional [G][trace_stride] wall-clock stamps (phase start, phase end, ...)
  int trace_stride;
  int stress;                 // 1: random delays before every arrival, NaN-poisoned exchange buffers
  // batched kernel: the normed phases' inputs, published by the O and down
  // phases: x times the next norm's gains in fp16 (8-row blocks, see blk8),
  // and each workgroup's partial sums of x^2 [G][kMaxBatch]
  uint16_t* xg16;
  float* ssp;
  Mailbox* mail;              // decode server mailbox (device address of host-pinned memory) or null
  float* lg_sys;              // decode server logits [B][Vlm] (device address of host-pinned memory) or null
  int32_t* srv_slot;          // decode server request slots [kSrvCopies][kMailRing][kReqWords]
  // mixture of experts (E > 0; F above is then topk * Fe, the down product's input)
  int E, topk, Fe;            // experts per layer, experts per token, expert width
  const uint8_t* w8;          // expert codes (E4M3): per layer Wgu8 [E][Fe][2][d], then Wd8 [E][d][Fe] at e8_d
  size_t e8_stride, e8_d;     // bytes between layers; offset of Wd8 inside a layer
  const float* esc;           // expert row scales: per layer [E][Fe][2] (gate, up), then [E][d] at sc_d
  size_t sc_stride, sc_d;     // floats between layers; offset of the down scales inside a layer
  int32_t* routes;            // chosen experts [max_ctx][L][topk]
  int mx;                     // 1: MXFP4 experts (w8 holds E2M1 pairs; xsc the E8M0 block scales)
  const uint8_t* xsc;         // MXFP4 scales: per layer Wgu [E][Fe][2][d/32], then Wd [E][d][Fe/32] at xsc_d
  size_t xsc_stride, xsc_d;   // bytes between layers; offset of the down scales inside a layer
  float* rpart;               // router logits' partial sums over each workgroup's rows [G][kMoeMaxExperts]
};

struct Launch {
  int pos0;          // position of the launch's first token
  int n_tok;         // tokens in this launch
  int tok_src;       // TOK_PROMPT (prompt[i]) or TOK_DEVICE (*tok_cur, then own argmax)
  int lm_last_only;  // LM head + argmax only for the last token (prefill)
  int write_logits;  // store the last token's logits
  int fenced;        // also issue agent-scope release/acquire fences at barriers
  uint32_t bar_base; // barriers completed before this launch (wrapping)
  int phase_begin;   // run only phases with global index in [phase_begin, phase_end)
  int phase_end;
  int pos_end;       // positions at or past pos_end are not computed (the ragged last step of a batched prefill)
  int n_force;       // 1: the first token's inputs are force[0..batch) instead of *tok_cur (teacher forcing)
  int force[kMaxBatch];
  int server;        // 1: token i is request i of P.mail; the launch ends where the mailbox closes
  uint32_t srv_epoch;     // tags this launch's request slots (never 0)
  uint32_t idle_ticks;    // workgroup 0 closes the mailbox after this long (wall clock) without a request
};

DEC_HD inline int phases_per_token(int L) { return kPhasesPerLayer * L + 2; }

// GEMV work splits, shared by the kernel and host-side checks.
// Items [b, e) of n for member g of G: contiguous, in order, sizes within one.
DEC_HD inline void split_even(int n, int g, int G, int& b, int& e) {
  b = (int)((long long)n * g / G);
  e = (int)((long long)n * (g + 1) / G);
}
// The batched kernel's 16-row groups of a GEMV over G workgroups, contiguous
// and in order, where the n mod G workgroups with one group more are the last
// ones: attention pairs go to the first workgroups, and the ones past them
// warm their gate/up tiles in the cache during attention, which hides the
// extra group there.
DEC_HD inline void split_tail(int n, int g, int G, int& b, int& e) {
  const int base = n / G, lo = G - n % G;   // workgroups [lo, G) take base + 1
  b = g < lo ? g * base : lo * base + (g - lo) * (base + 1);
  e = b + (g < lo ? base : base + 1);
}
// Piece columns of a GEMV row of K elements: 512 elements (64 lanes x 16 B) each.
DEC_HD inline int gemv_piece_cols(int K) { return (K + 511) >> 9; }
// Member s (1..n_members) of a workgroup's n units, where a unit is one piece
// column of one row pair and a pair's units are consecutive (npc of them):
// an even split, except that a boundary that would fall inside a row pair
// which already holds the previous boundary moves to that pair's end.  Then
// no row pair has more than two contributors, and two ds_add_f32 into a
// zeroed word give the same bits in either order.
DEC_HD inline void streamer_range(int n, int npc, int n_members, int s, int& u0, int& u1) {
  int prev = 0;
  u0 = u1 = 0;
  for (int k = 1; k <= n_members; ++k) {
    int b = (int)((long long)n * k / n_members);
    if (b < prev) b = prev;
    if (prev % npc != 0 && b / npc == prev / npc && b % npc != 0) b = (prev / npc + 1) * npc < n ? (prev / npc + 1) * npc : n;
    if (k == s) { u0 = prev; u1 = b; }
    prev = b;
  }
}

// Number of attention chunks per head at context length ctx for a grid of G
// workgroups and H heads (all sequences' heads in a batch): as many as keeps
// every wave of every workgroup busy (at most 8 G / H per head), no chunk
// shorter than kChunkMin positions, and at most kChunkCap chunks (one wave
// merges a head's partials) unless chunks would exceed kChunkMax positions.
constexpr int kChunkCap = 32;
DEC_HD inline int attn_chunks(int ctx, int H, int G) {
  int by_min = (ctx + kChunkMin - 1) / kChunkMin;
  int by_max = (ctx + kChunkMax - 1) / kChunkMax;
  int fill = 8 * G / H > 0 ? 8 * G / H : 1;
  int c = by_min < fill ? by_min : fill;
  c = c < kChunkCap ? c : kChunkCap;
  return c > by_max ? c : by_max;
}

DEC_HD inline int max_attn_chunks(int max_ctx, int H, int G) {
  int m = 1;
  // attn_chunks grows with ctx, so its value at max_ctx bounds every launch
  m = attn_chunks(max_ctx, H, G);
  return m < 1 ? 1 : m;
}

// Grid barriers a resident launch executes: one before every phase except the
// launch's first and a QKV phase that directly follows this launch's ARGMAX
// (each workgroup then already holds the token it computed itself).
inline uint32_t launch_barriers(int L, int n_tok, int lm_last_only) {
  uint32_t phases = 0, skipped = 0;
  for (int i = 0; i < n_tok; ++i) {
    bool lm = !lm_last_only || i == n_tok - 1;
    phases += kPhasesPerLayer * L + (lm ? 2 : 0);
    if (i > 0) {
      bool prev_lm = !lm_last_only || i - 1 == n_tok - 1;
      if (prev_lm) skipped += 1;
    }
  }
  return phases - 1 - skipped;
}

// Matrix-form prefill (dec_matrix.hip): the prompt's positions as the rows
// of matrix products on the matrix cores.  A product C = A B^T takes A
// [M x K] and B [N x K] fp16 with K contiguous and K a multiple of 32.
enum MpEpilogue : int {
  MP_EP_SCALE = 0,   // C = s[m] * (A B^T)  (s may be null: no scale)
  MP_EP_ACCUM = 1,   // C += A B^T
  MP_EP_PART = 2,    // internal: one K split's partial sums, [S][M][N]
  MP_EP_SWIGLU = 3,  // H[m][n/2] = fp16(silu(g) * u), g, u = s[m] (A B^T) at columns n, n+1 (n even)
  MP_EP_ROPE = 4,    // columns [q | k | v] of s[m] (A B^T): q, k rotated (q also times 1/sqrt(hd)),
                     // q to H (fp16 [M][ldh]), k and v to the fp16 cache at position pos0 + m
};
struct MpEpi {
  int mode;
  float* C; int ldc;           // SCALE, ACCUM, PART
  const float* s;              // row scales (SCALE, SWIGLU, ROPE; null: 1)
  uint16_t* H; int ldh;        // SWIGLU, ROPE: fp16 output rows
  const float* rope;           // ROPE: cos/sin table [max_ctx][hd/2][2]
  uint16_t* kc; uint16_t* vc;  // ROPE: the layer's K and V cache, [H][max_ctx][hd] each
  size_t head_elems;           // ROPE: max_ctx hd
  int pos0, q, hd;             // ROPE: position of row 0, H hd, head_dim
};
constexpr int kMpShapes = 6;           // tile shapes: 128x128, 128x64 (register-staged), 64x64, 128x64, 64x32 (LDS DMA), 16x64
constexpr int kMpChunk = 2048;         // prompt positions per pass over the weights
constexpr size_t kMpPartFloats = size_t(8) << 20;   // split-K partial sums buffer (floats)
struct MpGemm {
  const uint16_t* A; int lda;
  const uint16_t* B; int ldb;
  int M, N, K;
  MpEpi epi;                 // what becomes of each result (N even for the pair modes)
  int shape, S, kc;          // from mp_plan: tile shape, K splits, K elements per split
  float* part;               // [S][M][N] partial sums when S > 1
};
int mp_prepare();
void mp_plan(int M, int N, int K, size_t part_floats, int* shape, int* S, int* kc);
int mp_launch_embed(const uint16_t* E, const int* tok, int n, int d, float* x, void* stream);
int mp_launch_norm(const float* x, const float* g, int n, int d, float eps, uint16_t* h, float* s, void* stream);
int mp_launch_gemm(const MpGemm& g, void* stream);
int mp_launch_attention(const uint16_t* q16, int q, int n, int pos0, int H, int hd, const uint16_t* kc,
                        const uint16_t* vc, size_t head_elems, uint16_t* o16, void* stream);
int mp_launch_argmax(const float* logits, int V, int* tok_out, int* tok_cur, void* stream);

// Launch helpers defined next to the kernel (dec_kernels.hip).  P points to a
// device copy of the parameters; stream is a hipStream_t; batch selects the
// kernel built for one sequence or for up to kMaxBatch and hd the one built
// for that head dimension (8, 16, 32, 64 or 128); each returns a hipError_t
// value (0 = success; hipErrorInvalidValue for another head dimension).
// `kind` picks the resident kernel: the batch it is built for (1, or up to
// kMaxBatch for the batched one) or kMoeKernel (batch 1, mixture of experts)
int kernel_prepare();                                            // raise the dynamic-LDS limit
int kernel_blocks_per_cu(int kind, int hd, int* out);            // co-resident workgroups per CU
int kernel_launch_resident(const Params* P, const Launch& A, int grid, int kind, int hd, void* stream);  // cooperative
int kernel_launch_plain(const Params* P, const Launch& A, int grid, int kind, int hd, void* stream);     // ordinary
// Stream-ceiling read of n16 16-byte words at src on the null stream; out
// holds grid * kThreads words.
int kernel_stream_read(const void* src, uint64_t n16, uint32_t* out, int grid);
// Device address of the fixed no-allocation scratch array (kNoallocScratchBytes)
// on `device`, which must be the current device; looked up once per device.
int kernel_scratch(int device, void** out);

}  // namespace decmono
