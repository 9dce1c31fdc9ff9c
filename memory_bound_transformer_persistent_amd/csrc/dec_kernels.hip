// Resident decode kernel for gfx950 (MI355X).
//
// One launch runs whole decode steps: for every token, every layer's five
// phases (QKV GEMV, attention, O GEMV, gate/up GEMV, down GEMV), then the LM
// head and the greedy argmax.  Phases are separated by grid-wide barriers on
// device counters instead of kernel boundaries, which removes the per-launch
// cost and the host scheduling between operations that a one-kernel-per-op
// stack pays (hakusoku.com/story/7519, sections
// 標準推論スタックのボトルネックとKogの工夫 and Kog Inference Engineの特徴とイノベーション).
//
// Batch-1 decode reads every weight once per token through matrix-vector
// products, so it is bound by HBM bandwidth (same page, section
// GPU推論の速度制限要因：メモリ帯域幅).  Every GEMV streams its rows with 16-byte
// non-temporal buffer loads into registers (one 1 KB contiguous segment per
// wave instruction), reads its input vector from LDS, accumulates in fp32 and
// reduces across the wave with DPP.  No MFMA: at one token per step there is
// no dense contraction to feed it.  With several sequences at the same
// position (batch), the same pass over the weights serves all of them and the
// product is a skinny matrix multiply: the inputs sit in LDS as fp16, the
// weights are packed as 16 x 32 tiles, and each 1 KB tile is one
// v_mfma_f32_16x16x32_f16 against eight sequences' inputs.
//
// Cross-workgroup data (residual stream, q/k/v, attention partials, SwiGLU
// output, KV-cache appends, argmax partials) is written with agent-coherent
// (sc1) stores and read with agent-coherent loads, so a barrier needs no L2
// write-back or invalidate: a workgroup waits for its own stores to complete,
// then adds one to its group's counter; waiters poll the group counters.
// Weights are read-only for the whole launch and use plain non-temporal loads.
#include <hip/hip_runtime.h>
#include <math.h>

#include <mutex>

#include "dec_internal.h"

namespace decmono {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kAuxNt = 0x2;    // non-temporal: streamed once
constexpr int kAuxSc1 = 0x10;  // coherent at device (agent) scope
constexpr uint32_t kOOB = 0xFFFFFF00u;  // buffer offset past any region: loads read 0

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void;

// Roles: wave 0 controls (grid barrier, phase input vectors, global stores,
// attention, argmax); waves 1..7 stream GEMV weights into registers.
constexpr int kStreamers = kWaves - 1;
// Units (two 1 KB weight blocks) each streamer keeps in flight: 16-byte loads
// per lane land in registers, so a wave's LDS reads never queue behind its
// own weight traffic.
constexpr int kUnitsInFlight = 4;
constexpr int kBlocksInFlight = 2 * kUnitsInFlight;
// The batched kernel streams 1 KB weight tiles, one 16-byte load per lane each.
constexpr int kTilesInFlight = 8;
constexpr int kTabStride = 12;   // ints per (streamer, phase type) entry of the phase tables
constexpr int kStreamerTab = 6 * kTabStride;   // one streamer's entries: phase types 0..5
constexpr int kPlanInts = 32;    // per phase type: count, up to 2 * kStreamers combine entries; from 16 on the shared groups
constexpr int kAuxFloats = 2048;
// aux LDS: the step's rotary rows (up to 1024 floats; live from the QKV GEMV
// to the QKV publication) and, in the attention phase, the eight waves'
// attention partials (8 x (hd + 2) floats; live from the attention to its
// merge after S1) share offset 0: their lifetimes do not overlap
constexpr int kAuxPart = 0;
static_assert(kAuxPart + kWaves * (128 + 2) <= kAuxFloats, "aux LDS");
// Mixture of experts, in aux LDS the rotary rows and the attention partials
// leave free from the O phase to the down phase:
//   kAuxRouter  the router logits' sums over each wave's workgroups [8][64] (GU)
//   kAuxRoute   the layer's routing, 16 words per wave: the top_k experts
//               (ints), then their weights from word 8.  Each wave forms its
//               own copy in the GU phase; wave 0's is read until the down phase.
//   kAuxMoe     the down phase's row scales (kMoeScaleFloats)
constexpr int kAuxRouter = 0;
static_assert(kAuxRouter + kWaves * kMoeMaxExperts <= 1280, "aux LDS");
constexpr int kAuxRoute = 1280;
static_assert(kAuxRoute >= 1024 && kAuxRoute >= kAuxPart + kWaves * (128 + 2) && kAuxRoute + 16 * kWaves <= 1536,
              "aux LDS");

// LDS map (floats) for a kernel built for up to MB sequences:
// input region | out | xown | red | scales | si | aux | gains | phase tables |
// partial-output slots | combine plans | warm-up sink.
// MB == 1: the input region is the fp32 vector xs.  MB > 1: it holds the fp16
// inputs of every sequence side by side (stride = the phase's padded row
// length) and, for the normed phases, the fp32 residual vectors they come
// from, staged after them.
template <int MB>
struct Lds {
  static constexpr int Region = MB == 1 ? kMaxK : (kMaxBatch * kBatchSpanK) / 2;
  static constexpr int GainN = MB == 1 ? kMaxK : kBatchSpanD;
  static constexpr int Out = Region, Own = Out + kOutFloats, Red = Own + kOwnFloats;
  static constexpr int Scl = Red + kWaves * kMaxBatch, Si = Scl + kMaxBatch, Aux = Si + 16;
  static constexpr int Gain = Aux + kAuxFloats, TabWg = Gain + GainN, Tab = TabWg + 16;
  // batched kernel: a streamer's partial results for the (at most two)
  // 16-row output groups it shares with other streamers
  static constexpr int SlotN = MB == 1 ? 0 : kTileRows * MB;
  static constexpr int Slot = Tab + kStreamers * kStreamerTab, Plan = Slot + kStreamers * 2 * SlotN;
  // batch 1: 1 KB that the attention-phase cache warm-up DMAs land in (never read)
  static constexpr int Sink = Plan + (MB == 1 ? 0 : 6 * kPlanInts);
  // mixture of experts: the router's columns of the workgroup's residual
  // rows, fp16 [E][rows] (LDS DMA in the QKV phase, read by the O publication)
  static constexpr int MoeWr = Sink + 256;
  static constexpr int End = MoeWr + kMoeWrElems / 2;
  static_assert(End * 4 <= kLdsBytes, "LDS map exceeds the allocation");
  static_assert(MB == 1 || 3 * kMaxBatch * kBatchSpanD / 2 <= Region, "staged fp32 inputs do not fit");
  static_assert(Gain % 4 == 0 && Region % 4 == 0 && Sink % 4 == 0, "16-byte alignment");
  static_assert(Plan % 2 == 0 && kPlanInts % 2 == 0, "8-byte plan words (combine_all)");
};

constexpr int kWaitVm0 = 0x0F70;             // s_waitcnt vmcnt(0), expcnt/lgkmcnt untouched

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 ld_nt(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAuxNt);
}
__device__ __forceinline__ u32x4 ld_kv(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAuxNt | kAuxSc1);
}
// 16 bytes per lane from a buffer straight into LDS at lds_base + 16*lane (wave-uniform
// base), coherent at device scope (activations written by other workgroups).
__device__ __forceinline__ void dma16_coh(rsrc_t r, void* lds_base, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, off, 0, 0, kAuxSc1);
}
// Same for read-only data.
__device__ __forceinline__ void dma16_ld(rsrc_t r, void* lds_base, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, off, 0, 0, 0);
}
__device__ __forceinline__ void wait_vm0() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt[3:0] | expcnt 7 | lgkmcnt 15 | vmcnt[5:4] << 14)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
__device__ __forceinline__ void wait_lgkm0() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt/expcnt untouched
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Plain loads of read-only data through the global address space.
typedef __attribute__((address_space(1))) const float gfloat;
typedef __attribute__((address_space(1))) const int gint;
typedef __attribute__((address_space(1))) const f32x4 gf32x4;
__device__ __forceinline__ float ldg(const float* p) { return *(gfloat*)p; }
__device__ __forceinline__ int ldg(const int* p) { return *(gint*)p; }
__device__ __forceinline__ f32x4 ldg4(const float* p) { return *(gf32x4*)p; }
__device__ __forceinline__ f32x4 ld_coh4(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAuxSc1));
}
// Device-coherent (sc1) loads and stores of data other workgroups exchange,
// all through the global address space.  A flat access would also count in
// lgkmcnt, so every later scalar load or LDS read that waits for lgkmcnt
// would first wait for the store to be acknowledged.  A global access counts
// in vmcnt only, so several can be in flight and waited for in order.
typedef __attribute__((address_space(1))) float gfloat_rw;
typedef __attribute__((address_space(1))) int gint_rw;
typedef __attribute__((address_space(1))) uint32_t guint;
typedef __attribute__((address_space(1))) uint16_t gushort;
__device__ __forceinline__ float ld_coh(const float* p) {
  return __hip_atomic_load((gfloat_rw*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_coh(const int* p) {
  return __hip_atomic_load((gint_rw*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_coh(const uint32_t* p) {
  return __hip_atomic_load((guint*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(float* p, float v) {
  __hip_atomic_store((gfloat_rw*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(int* p, int v) {
  __hip_atomic_store((gint_rw*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(uint32_t* p, uint32_t v) {
  __hip_atomic_store((guint*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(uint16_t* p, uint16_t v) {
  __hip_atomic_store((gushort*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16 bytes per lane at byte offset off of buffer r, with the same
// device-scope (sc1) policy as st_coh
__device__ __forceinline__ void st_coh16(rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kAuxSc1);
}
// plain stores through the global address space (results the host reads)
typedef __attribute__((address_space(1))) uint64_t gu64;
__device__ __forceinline__ void st_g(float* p, float v) { *(gfloat_rw*)p = v; }
__device__ __forceinline__ void st_g(uint64_t* p, uint64_t v) { *(gu64*)p = v; }
__device__ __forceinline__ uint64_t ld_coh64(const uint64_t* p) {
  return __hip_atomic_load((gu64*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh64(uint64_t* p, uint64_t v) {
  __hip_atomic_store((gu64*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// System-scope accesses of host-pinned memory (the decode server's mailbox
// and logits), through the global address space
__device__ __forceinline__ int ld_sys(const int* p) {
  return __hip_atomic_load((gint_rw*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ uint32_t ld_sys(const uint32_t* p) {
  return __hip_atomic_load((guint*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void st_sys(int* p, int v) {
  __hip_atomic_store((gint_rw*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void st_sys(uint32_t* p, uint32_t v) {
  __hip_atomic_store((guint*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void st_sys(float* p, float v) {
  __hip_atomic_store((gfloat_rw*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
// Paths the decode steps never take unless asked for (decode server, debug
// modes, errors): marked unlikely so that the hot code is laid out densely
// (wave 0's serial code is instruction-cache bound; 1% at batch 8).
#define DEC_COLD(x) __builtin_expect(!!(x), 0)
// relaxed device-scope fetch-add, returning the old value
__device__ __forceinline__ uint32_t atomic_add_coh(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add((guint*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// wave reductions (DPP inside 16-lane rows, readlane across rows)
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// Every lane ends with the sum over its aligned group of LANES lanes (<= 16).
template <int LANES>
__device__ __forceinline__ float group_sum(float v) {
  if (LANES >= 2) v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  if (LANES >= 4) v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  if (LANES >= 8) v += dpp<0x141>(v);   // row_half_mirror
  if (LANES >= 16) v += dpp<0x140>(v);  // row_mirror
  return v;
}
__device__ __forceinline__ float readlane(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<16>(v);
  return (readlane(v, 0) + readlane(v, 16)) + (readlane(v, 32) + readlane(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  return fmaxf(fmaxf(readlane(v, 0), readlane(v, 16)), fmaxf(readlane(v, 32), readlane(v, 48)));
}

// 8 fp16 weights times 8 fp32 inputs, fp32 accumulate.
__device__ __forceinline__ float dot8(u32x4 w, f32x4 xa, f32x4 xb, float acc) {
  const f16x8 h = __builtin_bit_cast(f16x8, w);
  acc = __builtin_fmaf((float)h[0], xa[0], acc);
  acc = __builtin_fmaf((float)h[1], xa[1], acc);
  acc = __builtin_fmaf((float)h[2], xa[2], acc);
  acc = __builtin_fmaf((float)h[3], xa[3], acc);
  acc = __builtin_fmaf((float)h[4], xb[0], acc);
  acc = __builtin_fmaf((float)h[5], xb[1], acc);
  acc = __builtin_fmaf((float)h[6], xb[2], acc);
  acc = __builtin_fmaf((float)h[7], xb[3], acc);
  return acc;
}
__device__ __forceinline__ void split(int n, int g, int G, int& b, int& e) { split_even(n, g, G, b, e); }

// Columns of the batched kernel.  In a batched decode column b is sequence b
// and every column is at the token step's position.  In a batched prefill
// (cols_pos) the columns are kMaxBatch consecutive prompt positions of one
// sequence: column b of step i is position pos0 + kMaxBatch i + b, and all
// columns share that sequence's KV cache.
__device__ __forceinline__ int step_pos(const Params& P, const Launch& A, int i) {
  return A.pos0 + (P.cols_pos ? kMaxBatch * i : i);
}
__device__ __forceinline__ int col_pos(const Params& P, int pos, int b) { return P.cols_pos ? pos + b : pos; }
__device__ __forceinline__ int kv_seq(const Params& P, int b) { return P.cols_pos ? 0 : b; }
__device__ __forceinline__ int kv_heads(const Params& P) { return (P.cols_pos ? 1 : P.B) * P.H; }

// ---------------------------------------------------------------------------
// GEMV work and block streams
// ---------------------------------------------------------------------------
// A GEMV phase's work for one workgroup: row pairs [p0, p1) of W[rows, K].
// A row is NPC = ceil(K/512) piece-columns of 512 elements (64 lanes x 16 B);
// the workgroup's phase is the list of (pair, piece-column) units, unit
// n = pair_offset * NPC + column, and streamer s (1..7) takes an equal
// contiguous range of them.  A unit is two 1 KB blocks (row 0, row 1) that
// share one piece of x.  Partial row sums meet in LDS (ds_add_f32).
struct GemvWork {
  const uint16_t* W;
  int rows, K, p0, p1;
};

__device__ __forceinline__ int gemv_npc(int K) { return gemv_piece_cols(K); }
// Elements of the input vector a GEMV with row length K reads (zero-padded past K).
__device__ __forceinline__ int gemv_span(int K) { return 512 * gemv_npc(K); }
// Batched kernel: element (sequence b, row r) of the fp16 exchange vectors
// that several workgroups write and every workgroup pulls (the normed inputs
// and the SwiGLU output).  Blocks of 8 rows x kMaxBatch sequences are one
// 128-byte line each: a workgroup owns whole 16-row groups, so every line has
// one writer, and a publication store of 8 rows of all sequences fills one
// line.  Lines written by several workgroups took about twice as long to pull.
__device__ __forceinline__ size_t blk8(int b, int r) { return (size_t)(r >> 3) * (8 * kMaxBatch) + b * 8 + (r & 7); }

__device__ __forceinline__ GemvWork work_of(const Params& P, int ph, int l) {
  GemvWork g{nullptr, 0, 0, 0, 0};
  int npairs = 0;
  const uint16_t* lay = P.w + (size_t)l * P.layer_stride;
  switch (ph) {
    case PH_QKV: g.W = lay + P.off_qkv; g.rows = 3 * P.q; g.K = P.d; npairs = 3 * P.q / 2; break;
    case PH_O: g.W = lay + P.off_o; g.rows = P.d; g.K = P.q; npairs = P.d / 2; break;
    case PH_GU: g.W = lay + P.off_gu; g.rows = 2 * P.F; g.K = P.d; npairs = P.F; break;
    case PH_DOWN: g.W = lay + P.off_d; g.rows = P.d; g.K = P.F; npairs = P.d / 2; break;
    case PH_LM: g.W = P.w + P.off_lm; g.rows = P.Vlm; g.K = P.d; npairs = P.Vlm / 2; break;
    default: return g;
  }
  if (P.E > 0 && ph == PH_GU) {
    // mixture of experts: the GU phase streams only the chosen experts
    // (moe_stream), nothing through the ordinary stream
    g.p0 = g.p1 = 0;
    return g;
  }
  // batch 1 with few heads (at most 1/32 of the grid, e.g. one lane of a
  // tensor-parallel split): the workgroups that take attention (the first H)
  // get no QKV rows, so they reach the attention phase early and its K/V
  // history loads run while the others finish the QKV GEMV.  With more heads
  // the others' extra QKV rows cost more than this gains.
  const int G = gridDim.x, skip = (ph == PH_QKV && P.B == 1 && !P.cols_pos && P.H <= G / 32) ? P.H : 0;
  if ((int)blockIdx.x < skip) {
    g.p0 = g.p1 = 0;
  } else {
    split(npairs, blockIdx.x - skip, G - skip, g.p0, g.p1);
  }
  return g;
}

// Rows and row length of the matrix of GEMV phase type ph.
__device__ __forceinline__ void phase_shape(const Params& P, int ph, int& rows, int& K) {
  switch (ph) {
    case PH_QKV: rows = 3 * P.q; K = P.d; break;
    case PH_O: rows = P.d; K = P.q; break;
    case PH_GU: rows = 2 * P.F; K = P.d; break;
    case PH_DOWN: rows = P.d; K = P.F; break;
    default: rows = P.Vlm; K = P.d; break;
  }
}

// Streamer s's unit range [u0, u1) of a phase (streamer_range: no row pair
// has more than two contributors, so the partial sums do not depend on timing).
__device__ __forceinline__ void streamer_units(const GemvWork& g, int s, int& u0, int& u1) {
  const int npc = gemv_npc(g.K);
  streamer_range((g.p1 - g.p0) * npc, npc, kStreamers, s, u0, u1);
}

// Phase g of a launch: token i, layer l, phase type ph (-1: argmax, -2: not
// run, i.e. the LM head and argmax of a prefill token that wants no logits);
// k = g mod phases_per_token.  Decoded once per launch, then advanced.
struct PhaseIt { int g, i, k, l, ph; };
__device__ __forceinline__ int tail_phase(const Launch& A, int i, int k, int nl) {
  const bool lm = !A.lm_last_only || i == A.n_tok - 1;
  return !lm ? -2 : (k == nl ? (int)PH_LM : -1);
}
__device__ __forceinline__ PhaseIt phase_at(const Params& P, const Launch& A, int g) {
  const int ppt = phases_per_token(P.L), nl = kPhasesPerLayer * P.L;
  PhaseIt it;
  it.g = g;
  it.i = g / ppt;
  it.k = g - it.i * ppt;
  it.l = it.k < nl ? it.k / kPhasesPerLayer : 0;
  it.ph = it.k < nl ? it.k - it.l * kPhasesPerLayer : tail_phase(A, it.i, it.k, nl);
  return it;
}
__device__ __forceinline__ void phase_next(const Params& P, const Launch& A, PhaseIt& it) {
  const int nl = kPhasesPerLayer * P.L;
  ++it.g;
  if (++it.k == nl + 2) {
    it.k = 0; ++it.i; it.l = 0; it.ph = PH_QKV;
  } else if (it.k < nl) {
    if (++it.ph == kPhasesPerLayer) { it.ph = 0; ++it.l; }
  } else {
    it.l = 0;
    it.ph = tail_phase(A, it.i, it.k, nl);
  }
}
__device__ __forceinline__ bool is_gemv(int ph) {
  return ph == PH_QKV || ph == PH_O || ph == PH_GU || ph == PH_DOWN || ph == PH_LM;
}
// Phases whose input is rmsnorm(x) * g, and their g.
__device__ __forceinline__ bool norm_phase(const PhaseIt& id) {
  return id.ph == PH_QKV || id.ph == PH_GU || id.ph == PH_LM;
}
__device__ __forceinline__ const float* norm_gains(const Params& P, const PhaseIt& id) {
  if (id.ph == PH_LM) return P.gains + (size_t)P.L * 2 * P.d;
  return P.gains + (size_t)id.l * 2 * P.d + (id.ph == PH_GU ? P.d : 0);
}
// Row length of the GEMV of phase ph (its input's length).
__device__ __forceinline__ int phase_k(const Params& P, int ph) {
  return ph == PH_O ? P.q : (ph == PH_DOWN ? P.F : P.d);
}

// Launch-constant split of every GEMV phase type, computed once per launch
// into LDS (no divisions on the phase path).  Per type ph: the workgroup's
// pairs [p0, p1) (kept by wave 0) and, per streamer, its share of units.
enum TabField { T_LEFT, T_OFF, T_COL, T_NPC, T_ROWB, T_WRAP, T_TAIL, T_T0, T_NBYTES, T_PAD };
// wave 0's table: (p0, p1) per phase type in ints 0..11; a mixture of
// experts' slot, q0, q1 (moe_slot) from int kTabMoeSlot on
constexpr int kTabMoeSlot = 12;

__device__ __forceinline__ int rfl(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Batched kernel: a workgroup owns whole 16-row groups [g0, g1) of each
// matrix (its row pairs for the publisher: [8 g0, min(8 g1, rows/2))) and its
// tiles, g0*KT .. g1*KT-1 in the tiled image, are one contiguous byte range
// that the streamers split evenly.  Per streamer: T_LEFT tiles from byte
// T_OFF, the first one in the workgroup's row group T_T0 at k-tile T_COL of
// T_NPC; T_NBYTES bounds the matrix; T_PAD rounds to whole groups.
__device__ __forceinline__ void fill_tables_tiled(const Params& P, int wave, int* tab_wg, int* tab) {
  const int lane = threadIdx.x & 63;
  if (lane >= 6 || lane == PH_ATTN) return;
  int rows, K;
  phase_shape(P, lane, rows, K);
  const int rg = (rows + kTileRows - 1) / kTileRows, kt = (K + kTileCols - 1) / kTileCols;
  int g0, g1;
  split_tail(rg, blockIdx.x, gridDim.x, g0, g1);
  if (wave == 0) {
    tab_wg[2 * lane] = (kTileRows / 2) * g0;
    tab_wg[2 * lane + 1] = min((kTileRows / 2) * g1, rows / 2);
    return;
  }
  int u0, u1;
  split((g1 - g0) * kt, wave - 1, kStreamers, u0, u1);
  int* e = tab + lane * kTabStride;
  e[T_LEFT] = u1 - u0;
  e[T_OFF] = (int)((uint32_t)(g0 * kt + u0) * 1024u);
  e[T_COL] = u0 % kt;
  e[T_NPC] = kt;
  e[T_T0] = u0 / kt;
  e[T_NBYTES] = (int)((uint32_t)(rg * kt) * 1024u);
  e[T_PAD] = (kTilesInFlight - (u1 - u0) % kTilesInFlight) % kTilesInFlight;
}

// Mixture of experts: the expert slot of workgroup b (slot floor(b top_k /
// G), so every slot has G / top_k workgroups or one more) and its gate/up row
// pairs [q0, q1) of the slot's expert (an even split of Fe over the slot's
// workgroups).
__device__ __forceinline__ void moe_slot(const Params& P, int b, int G, int& slot, int& q0, int& q1) {
  slot = (int)((long long)b * P.topk / G);
  const int first = (int)(((long long)slot * G + P.topk - 1) / P.topk);
  const int next = (int)(((long long)(slot + 1) * G + P.topk - 1) / P.topk);
  split(P.Fe, b - first, next - first, q0, q1);
}

__device__ __forceinline__ void fill_tables(const Params& P, int wave, int* tab_wg, int* tab) {
  const int lane = threadIdx.x & 63;
  if (lane >= 6 || lane == PH_ATTN) return;
  GemvWork w = work_of(P, lane, 0);
  if (wave == 0) {
    tab_wg[2 * lane] = w.p0;
    tab_wg[2 * lane + 1] = w.p1;
    if (P.E > 0 && lane == 0) moe_slot(P, blockIdx.x, gridDim.x, tab_wg[kTabMoeSlot], tab_wg[kTabMoeSlot + 1],
                                       tab_wg[kTabMoeSlot + 2]);
    return;
  }
  // mixture of experts: the down phase's rows are streamed once the routing
  // is known (moe_stream), not by the cursor
  if (P.E > 0 && lane == PH_DOWN) w.p1 = w.p0;
  int u0, u1;
  streamer_units(w, wave, u0, u1);
  const uint32_t npc = (uint32_t)gemv_npc(w.K), rowb = (uint32_t)w.K * 2u;
  int* e = tab + lane * kTabStride;   // tab: this streamer's entries
  const int t0 = u0 / (int)npc, col = u0 - t0 * (int)npc;
  e[T_LEFT] = u1 - u0;
  e[T_OFF] = (int)((uint32_t)(2 * (w.p0 + t0)) * rowb + 1024u * (uint32_t)col);
  e[T_COL] = col;
  e[T_NPC] = (int)npc;
  e[T_ROWB] = (int)rowb;
  e[T_WRAP] = (int)(2u * rowb - 1024u * (npc - 1));   // last column -> next pair's column 0
  e[T_TAIL] = (int)((uint32_t)(w.K >> 3) - 64u * (npc - 1));   // lanes with data in the last column
  e[T_T0] = t0;
  e[T_NBYTES] = (int)((uint32_t)w.rows * rowb);
  // zero-reading units that round the phase up to whole groups of kUnitsInFlight
  e[T_PAD] = (kUnitsInFlight - (u1 - u0) % kUnitsInFlight) % kUnitsInFlight;
}

// Deterministic partial sums in the batched kernel, where a 16-row group's
// tiles are usually split over several streamers.  A group that one streamer
// computes entirely is stored by it directly.  A group several streamers
// share (only the first or last group of a streamer's range can be shared)
// is stored by each of them in its own slot, and after the phase all eight
// waves add the slots in streamer order (combine_all): the result does not
// depend on which streamer finished first.  The plan lists, per phase type,
// the shared (streamer, end) slots in that order (an entry is slot | group <<
// 4 | (first slot of its group) << 28), and from int 16 on the count of
// shared groups, then from int 18 two ints per shared group: output group |
// slot count << 8, and its slots, 4 bits each in streamer order (a group has
// at most one slot per streamer, so at most kStreamers).
__device__ __forceinline__ bool whole_group(int t, int kt, int u0, int u1) { return t * kt >= u0 && (t + 1) * kt <= u1; }

__device__ __forceinline__ void build_plans(const int* tab_all, int* plan) {
  const int lane = threadIdx.x & 63;
  if (lane >= 6 || lane == PH_ATTN) return;
  int cnt = 0, prev = -1;
  int* pl = plan + lane * kPlanInts;
  for (int s = 0; s < kStreamers; ++s) {
    const int* e = tab_all + (s * 6 + lane) * kTabStride;
    const int n = e[T_LEFT];
    if (n <= 0) continue;
    const int kt = e[T_NPC], t0 = e[T_T0], u0 = t0 * kt + e[T_COL], u1 = u0 + n, t1 = (u1 - 1) / kt;
    for (int w = 0; w < 2; ++w) {
      const int t = w == 0 ? t0 : t1;
      if (w == 1 && t1 == t0) break;
      if (whole_group(t, kt, u0, u1)) continue;
      pl[1 + cnt] = (s * 2 + w) | (t << 4) | ((t != prev ? 1 : 0) << 28);
      prev = t;
      ++cnt;
    }
  }
  pl[0] = cnt;
  // the shared groups: output group, slot count and slot list of each
  int* gp = pl + 16;
  int ng = 0;
  for (int k = 0; k < cnt; ++k) {
    const int en = pl[1 + k];
    if ((en >> 28) & 1) {
      gp[2 + 2 * ng] = ((en >> 4) & 0xFF) | (1 << 8);
      gp[3 + 2 * ng] = en & 15;
      ++ng;
    } else if (ng > 0) {
      const int c = gp[2 * ng] >> 8;
      gp[2 * ng] += 1 << 8;
      gp[2 * ng + 1] |= (en & 15) << (4 * c);
    }
  }
  gp[0] = ng;
}

// All eight waves, after the streamers have stored a batched phase's results
// (S2): out[group] = the sum of its shared slots, added in streamer order
// (the first slot's value, then each later one), one (group, element) per
// thread.
template <int MB>
__device__ __forceinline__ void combine_all(int ph, const int* plan, const float* slots, float* out) {
  constexpr int SN = Lds<MB>::SlotN;
  const int* gp = plan + ph * kPlanInts + 16;
  const int n = gp[0] * SN;
  for (int p = threadIdx.x; p < n; p += kThreads) {
    const int gi = p / SN, e = p - gi * SN;
    // one read for the group's slots, then all its slot reads at once
    const int2 d = *reinterpret_cast<const int2*>(gp + 2 + 2 * gi);
    const int g = d.x & 0xFF, ne = d.x >> 8;
    float v[kStreamers];
#pragma unroll
    for (int k = 0; k < kStreamers; ++k) v[k] = k < ne ? slots[((d.y >> (4 * k)) & 15) * SN + e] : 0.f;
    float acc = v[0];
#pragma unroll
    for (int k = 1; k < kStreamers; ++k)
      if (k < ne) acc += v[k];
    out[g * SN + e] = acc;
  }
}

__device__ __forceinline__ void lds_add(float* p, float v) {
  __builtin_amdgcn_ds_faddf((__attribute__((address_space(3))) float*)p, v, 0, 0, false);
}

__device__ __forceinline__ const uint16_t* gemv_base(const Params& P, int ph, int l) {
  const uint16_t* lay = P.w + (size_t)l * P.layer_stride;
  switch (ph) {
    case PH_QKV: return lay + P.off_qkv;
    case PH_O: return lay + P.off_o;
    case PH_GU: return lay + P.off_gu;
    case PH_DOWN: return lay + P.off_d;
    default: return P.w + P.off_lm;
  }
}

// A streamer's position in its block stream (wave-uniform).  The next unit is
// column col of the pair whose row 0 starts at byte `off` of phase it's
// matrix; `left` units of the phase remain, then `pad` zero-reading ones
// that round the phase to whole groups.  Once the stream has ended every
// further load is out of range and reads zeros, so the number of loads in
// flight never changes.
struct Cursor {
  PhaseIt it;
  uint32_t left, pad, off, col, npc, row_bytes, wrap, tail;
  rsrc_t r;
};

// Take phase it if this streamer has units in it.
__device__ __forceinline__ bool cursor_take(const Params& P, const int* tab, Cursor& cu) {
  if (!is_gemv(cu.it.ph)) return false;
  const int* e = tab + cu.it.ph * kTabStride;
  const int left = rfl(e[T_LEFT]);
  if (left <= 0) return false;
  cu.left = (uint32_t)left;
  cu.pad = (uint32_t)rfl(e[T_PAD]);
  cu.off = (uint32_t)rfl(e[T_OFF]);
  cu.col = (uint32_t)rfl(e[T_COL]);
  cu.npc = (uint32_t)rfl(e[T_NPC]);
  cu.row_bytes = (uint32_t)rfl(e[T_ROWB]);
  cu.wrap = (uint32_t)rfl(e[T_WRAP]);
  cu.tail = (uint32_t)rfl(e[T_TAIL]);
  // phase and layer through readfirstlane: the Params fields gemv_base reads
  // then come from scalar loads, not a vector load that would wait for every
  // weight load in flight
  cu.r = make_rsrc(gemv_base(P, rfl(cu.it.ph), rfl(cu.it.l)), (uint32_t)rfl(e[T_NBYTES]));
  return true;
}
__device__ __forceinline__ void cursor_start(const Params& P, const Launch& A, int g0, int g1, const int* tab,
                                             Cursor& cu) {
  cu.left = cu.pad = 0;
  cu.col = cu.npc = cu.off = cu.row_bytes = cu.wrap = cu.tail = 0;
  cu.r = make_rsrc(P.w, 0);
  if (g0 >= g1) { cu.it.g = g1; return; }
  cu.it = phase_at(P, A, g0);
  while (!cursor_take(P, tab, cu)) {
    phase_next(P, A, cu.it);
    if (cu.it.g >= g1) return;
  }
}
__device__ __forceinline__ void cursor_next(const Params& P, const Launch& A, int g1, const int* tab, Cursor& cu) {
  do {
    phase_next(P, A, cu.it);
    if (cu.it.g >= g1) return;
  } while (!cursor_take(P, tab, cu));
}

// Load the cursor's next unit (both rows, 16 B per lane each); advance.
// Straight-line code: the two loads are the same instructions whatever the
// cursor's state, so their destination registers never need copying.
__device__ __forceinline__ void issue_unit(Cursor& cu, uint32_t lane16, u32x4& b0, u32x4& b1) {
  const bool live = cu.left > 0;
  const bool last_col = cu.col + 1 == cu.npc;
  const bool ok = live && (!last_col || (lane16 >> 4) < cu.tail);
  const uint32_t o0 = ok ? cu.off + lane16 : kOOB;
  const uint32_t o1 = ok ? cu.off + cu.row_bytes + lane16 : kOOB + 16u;   // distinct: always two loads
  b0 = ld_nt(cu.r, o0);
  b1 = ld_nt(cu.r, o1);
  cu.left -= live ? 1u : 0u;
  cu.pad -= (!live && cu.pad > 0) ? 1u : 0u;
  cu.off += live ? (last_col ? cu.wrap : 1024u) : 0u;
  cu.col = live ? (last_col ? 0u : cu.col + 1u) : cu.col;
}

// Tile stream of the batched kernel: a streamer's tiles of a phase are
// consecutive 1 KB blocks, so its cursor is a byte offset and a count.
struct TileCursor {
  PhaseIt it;
  uint32_t left, pad, off;
  rsrc_t r;
};
__device__ __forceinline__ bool tcursor_take(const Params& P, const int* tab, TileCursor& cu) {
  if (!is_gemv(cu.it.ph)) return false;
  const int* e = tab + cu.it.ph * kTabStride;
  const int left = rfl(e[T_LEFT]);
  if (left <= 0) return false;
  cu.left = (uint32_t)left;
  cu.pad = (uint32_t)rfl(e[T_PAD]);
  cu.off = (uint32_t)rfl(e[T_OFF]);
  cu.r = make_rsrc(gemv_base(P, rfl(cu.it.ph), rfl(cu.it.l)), (uint32_t)rfl(e[T_NBYTES]));
  return true;
}
__device__ __forceinline__ void tcursor_start(const Params& P, const Launch& A, int g0, int g1, const int* tab,
                                              TileCursor& cu) {
  cu.left = cu.pad = cu.off = 0;
  cu.r = make_rsrc(P.w, 0);
  if (g0 >= g1) { cu.it.g = g1; return; }
  cu.it = phase_at(P, A, g0);
  while (!tcursor_take(P, tab, cu)) {
    phase_next(P, A, cu.it);
    if (cu.it.g >= g1) return;
  }
}
__device__ __forceinline__ void tcursor_next(const Params& P, const Launch& A, int g1, const int* tab,
                                             TileCursor& cu) {
  do {
    phase_next(P, A, cu.it);
    if (cu.it.g >= g1) return;
  } while (!tcursor_take(P, tab, cu));
}
// Load the cursor's next tile into slot k (16 B per lane); advance.  Past the
// stream's end the load is out of range (a distinct offset per slot) and reads 0.
__device__ __forceinline__ void issue_tile(TileCursor& cu, uint32_t lane16, int k, u32x4& b) {
  const bool live = cu.left > 0;
  b = ld_nt(cu.r, live ? cu.off + lane16 : kOOB + 16u * (uint32_t)k);
  cu.left -= live ? 1u : 0u;
  cu.pad -= (!live && cu.pad > 0) ? 1u : 0u;
  cu.off += live ? 1024u : 0u;
}


// ---------------------------------------------------------------------------
// wave 0: grid barrier
// ---------------------------------------------------------------------------
// Arrive: wave 0 has issued every coherent store of the phase; it waits for
// them, then adds one to its group's counter (group = blockIdx % 8) and waits
// for that atomic too, so its first poll does not race its own arrival into
// the memory system (1% faster than polling at once).  Wait:
// lanes 0..7 poll the eight group counters until each holds
// group_size * epoch (epoch = cumulative barrier number, wrapping).  Returns
// false if the watchdog expires or any workgroup raised an error.
__device__ __forceinline__ void w0_arrive(const Params& P, int fenced) {
  wait_vm0();
  if ((threadIdx.x & 63) == 0) {
    if (DEC_COLD(fenced)) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t old = atomic_add_coh(P.ctl + kCtlGroup0 + 64 * (blockIdx.x % kGroups), 1u);
    __asm__ volatile("" ::"v"(old));
  }
  // the atomic has landed before the first poll goes out
  wait_vm0();
}

__device__ __forceinline__ bool w0_wait(const Params& P, uint32_t epoch, int fenced) {
  const int lane = threadIdx.x & 63;
  const uint32_t G = gridDim.x;
  const int ng = G < (uint32_t)kGroups ? (int)G : kGroups;
  uint32_t target = 0;
  // lanes 0..ng-1 watch the group counters and lane kGroups the error word,
  // all in one load, so each poll costs one round trip
  const uint32_t* w = lane < ng ? P.ctl + kCtlGroup0 + 64 * lane : (lane == kGroups ? P.ctl + kCtlErr : P.ctl + kCtlGroup0);
  if (lane < ng) target = ((G - (uint32_t)lane + kGroups - 1) / kGroups) * epoch;
  const uint64_t t0 = wall_clock64();
  const uint64_t limit = (uint64_t)P.watchdog_ticks;
  // 0 = released, 1 = a workgroup raised an error, 2 = the watchdog expired
  int why = 0;
  while (true) {
    const uint32_t v = ld_coh(w);
    if (__any(lane == kGroups && v != 0u)) { why = 1; break; }
    if (__all(lane >= ng || (int)(v - target) >= 0)) break;
    if (wall_clock64() - t0 > limit) { why = 2; break; }
  }
  if (why == 2 && lane == 0) {
    uint32_t expected = 0u;
    __hip_atomic_compare_exchange_strong((guint*)(P.ctl + kCtlErr), &expected, (uint32_t)kDevErrTimeout, __ATOMIC_RELAXED,
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const bool ok = why == 0;
  if (DEC_COLD(fenced)) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  // no load the caller issues after the release moves above the poll loop
  // (the loads themselves are device-coherent and issue in program order)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return ok;
}

// ---------------------------------------------------------------------------
// stress mode (a debug aid for the barrier)
// ---------------------------------------------------------------------------
// A workgroup waits a pseudo-random 0 to about 2 us before each arrival, so
// the order in which workgroups arrive and read each phase's inputs varies
// from barrier to barrier.  The wait is bounded and wave-uniform.
__device__ __forceinline__ void stress_delay(uint32_t epoch) {
  uint32_t h = (blockIdx.x + 1u) * 2654435761u ^ epoch * 0x9E3779B9u;
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  const int n = rfl((int)(h % 12u));
  for (int i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(8);   // 8 x 64 cycles each
}

// Once the barrier before phase ph (layer l) has released this workgroup,
// fill with NaN the exchange buffers (or this workgroup's share of them)
// whose readers have all passed that barrier and whose next writer runs after
// a later one; none of them is phase ph's own input.  A reader that saw a
// value before the write meant for it was visible would read NaN (or, for
// token indices, -1), and the logits or tokens would show it.
template <int MB>
__device__ __forceinline__ void w0_poison(const Params& P, int ph, int l, const int* tab_wg) {
  const int lane = threadIdx.x & 63, G = gridDim.x, B = P.B;
  const uint32_t nan32 = 0x7FC00000u;
  const uint16_t nan16 = 0x7E00u;
  auto share = [&](int n, int& a, int& e) { split(n, blockIdx.x, G, a, e); };
  int a, e;
  if (ph == PH_ATTN || ph == PH_DOWN) {
    // residual rows this workgroup publishes next (in O, resp. DOWN); their
    // readers, the QKV (resp. GU) input pulls, are behind the barrier
    int r0, r1;
    own_rows<MB>(P, r0, r1);
    for (int b = 0; b < B; ++b)
      for (int r = r0 + lane; r < r1; r += 64) st_coh(reinterpret_cast<uint32_t*>(P.x + (size_t)b * P.d + r), nan32);
    if constexpr (MB > 1) {
      // and the normed inputs published with them
      for (int b = 0; b < B; ++b)
        for (int r = r0 + lane; r < r1; r += 64) st_coh(P.xg16 + blk8(b, r), nan16);
      if (lane < MB) st_coh(reinterpret_cast<uint32_t*>(P.ssp + (size_t)blockIdx.x * kMaxBatch + lane), nan32);
    }
  }
  if (ph == PH_QKV) {
    // this workgroup's SwiGLU outputs, read by the last DOWN input pull; GU
    // publishes them next (a mixture of experts: its slot's part)
    const bool moe = MB == 1 && P.E > 0;
    const int base = moe ? rfl(tab_wg[kTabMoeSlot]) * P.Fe : 0;
    const int p0 = base + rfl(tab_wg[moe ? kTabMoeSlot + 1 : 2 * PH_GU]);
    const int p1 = base + rfl(tab_wg[moe ? kTabMoeSlot + 2 : 2 * PH_GU + 1]);
    for (int b = 0; b < B; ++b)
      for (int t = p0 + lane; t < p1; t += 64) {
        if constexpr (MB == 1) st_coh(reinterpret_cast<uint32_t*>(P.act + t), nan32);
        else st_coh(P.act16 + blk8(b, t), nan16);
      }
  }
  if (ph == PH_O) {
    // q and the attention partials, read during the attention phase
    share(B * P.q, a, e);
    for (int i = a + lane; i < e; i += 64) {
      const int b = i / P.q;
      st_coh(reinterpret_cast<uint32_t*>(P.qkv + (size_t)b * 3 * P.q + (i - b * P.q)), nan32);
    }
    const int nparts = B * P.H * P.max_chunks;   // the partial slots the attention phase uses
    share(nparts * P.hd, a, e);
    for (int i = a + lane; i < e; i += 64) st_coh(reinterpret_cast<uint32_t*>(P.part + i), nan32);
    share(nparts * 2, a, e);
    for (int i = a + lane; i < e; i += 64) st_coh(reinterpret_cast<uint32_t*>(P.pml + i), nan32);
  }
  if (MB == 1 && P.E > 0 && ph == PH_DOWN && lane < P.E) {
    // mixture of experts: this workgroup's router-logit shares, read by every
    // workgroup's GU phase (behind the barrier); the next O publication writes them
    st_coh(reinterpret_cast<uint32_t*>(P.rpart + (size_t)blockIdx.x * kMoeMaxExperts + lane), nan32);
  }
  if (ph == PH_GU) {
    // the attention output, read by the O input pull
    share(B * P.q, a, e);
    for (int i = a + lane; i < e; i += 64) {
      if constexpr (MB == 1) st_coh(reinterpret_cast<uint32_t*>(P.att_o + i), nan32);
      else st_coh(P.att_o16 + i, nan16);
    }
  }
  if (ph == PH_ATTN && l == 0) {
    // argmax partials, read by the previous token's ARGMAX phase, which no
    // barrier separates from this token's QKV phase
    share((MB == 1 ? 1 : kMaxBatch) * G, a, e);
    for (int i = a + lane; i < e; i += 64) {
      st_coh(reinterpret_cast<uint32_t*>(P.amax_v + i), nan32);
      st_coh(P.amax_i + i, -1);
    }
  }
}

// ---------------------------------------------------------------------------
// phase inputs
// ---------------------------------------------------------------------------
// RMSNorm is split so that no wave waits on a reduction before the GEMV:
// wave 0 lands the raw vector(s) and the norm gains in LDS (LDS DMA); all
// waves then form x * g and their shares of sum(x^2); the scalar
// 1/sqrt(mean(x^2) + eps) multiplies the phase's outputs when wave 0
// publishes them, since W (x g s) = s W (x g).

// dst[0..gemv_span(n) elements of esize bytes) <- src[0..n) by LDS DMA
// (coherent when coh; zero past n).  Issues only; the caller waits.
// extra: that many more elements of zero fill past n (rounded up to 512)
__device__ __forceinline__ void w0_dma_vec(void* dst, const void* src, int n, int esize, bool coh, int extra = 0) {
  const int lane = threadIdx.x & 63;
  const rsrc_t r = make_rsrc(src, (uint32_t)(n * esize));
  const int span_bytes = gemv_span(n + extra) * esize;
  for (int o = 0; o < span_bytes; o += 1024) {
    void* base = static_cast<char*>(dst) + o;
    if (coh) dma16_coh(r, base, (uint32_t)(o + 16 * lane));
    else dma16_ld(r, base, (uint32_t)(o + 16 * lane));
  }
}

// Batched kernel: does phase id take its raw input vectors by LDS DMA (all
// but the attention, the argmax and layer 0's embedded QKV input)?
__device__ __forceinline__ bool dma_input(const PhaseIt& id) {
  return id.ph == PH_GU || id.ph == PH_LM || id.ph == PH_DOWN || id.ph == PH_O || (id.ph == PH_QKV && id.l > 0);
}
// Batched kernel, wave w of the workgroup: its share (1 KB chunks w, w + 8,
// ...) of phase id's fp16 input into the input region, in 8-row blocks as
// blk8 lays them out (so that a lane's MFMA B operand, 8 consecutive columns
// of one sequence, is 16 contiguous bytes), zero past row n: the normed
// phases' x times gains and the SwiGLU output are copied as they are; the
// attention output, [B][q] in memory, is gathered (each load still reads 8
// whole 128-byte runs).  Issues only; the caller waits.
template <int MB>
__device__ __forceinline__ void dma_input_share(const Params& P, const PhaseIt& id, float* xs, int w) {
  const int lane = threadIdx.x & 63;
  const bool normed = id.ph != PH_DOWN && id.ph != PH_O;
  const int n = normed ? P.d : (id.ph == PH_DOWN ? P.F : P.q);
  // 1 KB chunk c holds rows 64c .. 64c + 63 of every sequence (n is a
  // multiple of 8, so a lane's 16 bytes are all in range or all past it)
  const int nch = gemv_span(n) * 2 * kMaxBatch >> 10;
  char* base = reinterpret_cast<char*>(xs);
  if (id.ph == PH_O) {
    const rsrc_t r = make_rsrc(P.att_o16, (uint32_t)(P.B * n * 2));
    const int b = lane & (kMaxBatch - 1);
    for (int c = w; c < nch; c += kWaves) {
      const int row = 64 * c + 8 * (lane >> 3);
      dma16_coh(r, base + 1024 * c, b < P.B && row < n ? (uint32_t)((b * n + row) * 2) : kOOB);
    }
    return;
  }
  const rsrc_t r = make_rsrc(normed ? P.xg16 : P.act16, (uint32_t)(n * 2 * kMaxBatch));
  for (int c = w; c < nch; c += kWaves) dma16_coh(r, base + 1024 * c, (uint32_t)(1024 * c + 16 * lane));
}

// Batched kernel, wave w, a normed phase whose input was published by the O
// or down phase: red[b * kWaves + w] <- the sum of workgroups w*8 + j, j +=
// 64, of their partial sums of x^2 of sequence b (fixed order).
__device__ __forceinline__ void ss_share(const Params& P, int w, float* red) {
  const int lane = threadIdx.x & 63, b = lane & (kMaxBatch - 1);
  float ss = 0.f;
  for (int g = w * 8 + (lane >> 3); g < (int)gridDim.x; g += 64) ss += ld_coh(P.ssp + (size_t)g * kMaxBatch + b);
  ss += __shfl_xor(ss, 8, 64);
  ss += __shfl_xor(ss, 16, 64);
  ss += __shfl_xor(ss, 32, 64);
  if (lane < kMaxBatch) red[lane * kWaves + w] = ss;
}

// MB == 1, all waves: xs[0..n) *= gs[0..n); red[wave] <- this wave's share of sum(x^2).
__device__ __forceinline__ void apply_gains(float* xs, const float* gs, int n, float* red) {
  float ss = 0.f;
  for (int i = 4 * (int)threadIdx.x; i < n; i += 4 * kThreads) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(xs + i);
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    *reinterpret_cast<f32x4*>(xs + i) = v * *reinterpret_cast<const f32x4*>(gs + i);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
}

// MB > 1, all waves: for each sequence b, xh[b][0..span) <- fp16(st[b] * gs)
// (st: the staged fp32 vectors, zero past n) and red[b*kWaves + wave] <- this
// wave's share of sum(st[b]^2).
__device__ __forceinline__ void apply_gains_batch(_Float16* xh, const float* st, const float* gs, int n, int B,
                                                  float* red) {
  const int span = gemv_span(n);
  for (int b = 0; b < B; ++b) {
    float ss = 0.f;
    for (int i = 4 * (int)threadIdx.x; i < span; i += 4 * kThreads) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(st + (size_t)b * span + i);
      ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
      const f32x4 y = v * *reinterpret_cast<const f32x4*>(gs + i);
      // 8-row blocks as the pulled inputs (blk8); i is a multiple of 4
      *reinterpret_cast<f16x4*>(xh + blk8(b, i)) = f16x4{(_Float16)y[0], (_Float16)y[1], (_Float16)y[2], (_Float16)y[3]};
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[b * kWaves + (threadIdx.x >> 6)] = ss;
  }
}

// The rows [r0, r1) of the residual stream this workgroup owns: the rows it
// computes in the O and down phases (row pairs at batch 1, whole 16-row
// groups in the batched kernel).
template <int MB>
__device__ __forceinline__ void own_rows(const Params& P, int& r0, int& r1) {
  if constexpr (MB == 1) {
    int p0, p1;
    split(P.d / 2, blockIdx.x, gridDim.x, p0, p1);
    r0 = 2 * p0;
    r1 = 2 * p1;
  } else {
    int g0, g1;
    split_tail((P.d + kTileRows - 1) / kTileRows, blockIdx.x, gridDim.x, g0, g1);
    r0 = min(P.d, kTileRows * g0);
    r1 = min(P.d, kTileRows * g1);
  }
}

// Layer-0 input of sequence b: x = E[tok] (fp16 -> fp32) into dst (raw, zero
// past d).  This workgroup's rows of x go to xown (own floats per sequence)
// and to global x.
template <int MB>
__device__ __forceinline__ void w0_embed(const Params& P, int b, int tok, float* dst, float* xown, int own) {
  const int lane = threadIdx.x & 63, d = P.d;
  const _Float16* e = reinterpret_cast<const _Float16*>(P.w + P.off_E + (size_t)tok * d);
  int r0, r1;
  own_rows<MB>(P, r0, r1);
  const int span = gemv_span(d);
  for (int i = 8 * lane; i < span; i += 512) {
    f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
    if (i < d) {
      const f16x8 h = __builtin_bit_cast(f16x8, ldg4(reinterpret_cast<const float*>(e + i)));
      lo = f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
      hi = f32x4{(float)h[4], (float)h[5], (float)h[6], (float)h[7]};
    }
    *reinterpret_cast<f32x4*>(dst + i) = lo;
    *reinterpret_cast<f32x4*>(dst + i + 4) = hi;
  }
  wait_lgkm0();
  for (int r = r0 + lane; r < r1; r += 64) {
    xown[b * own + r - r0] = dst[r];
    st_coh(P.x + (size_t)b * d + r, dst[r]);
  }
}

// ---------------------------------------------------------------------------
// attention
// ---------------------------------------------------------------------------
// Single-query attention of every (column, head) pair over its positions
// 0..pos_b.  The QKV phase has already rotated and scaled q and appended this
// step's keys and values to the cache, so attention reads q and cached rows
// only.  A pair's positions are cut into chunks; each wave of the pair's
// workgroups runs an online softmax over one chunk (attend_chunk), the
// partials (max m, sum of exp l, sum of exp * V) of a workgroup's waves meet
// in LDS, and the workgroups of a pair meet through memory and an arrival
// counter: o = sum_c e^(m_c - M) acc_c / sum_c e^(m_c - M) l_c.

// The last arrival of pair hb (column, head): reset its counter, merge its C
// partials with a running max and store o at o_at.  Lane k owns dims 2k, 2k+1.
template <int MB>
__device__ __forceinline__ void merge_head(const Params& P, int hb, int C, size_t o_at) {
  const int lane = threadIdx.x & 63, hd = P.hd;
  if (lane == 0) st_coh(P.ctl + kCtlHead0 + hb, 0u);
  const int dd = 2 * lane;
  const bool act = dd < hd;
  const float* pbase = P.part + (size_t)hb * P.max_chunks * hd + (act ? dd : 0);
  const float* mbase = P.pml + (size_t)hb * P.max_chunks * 2;
  float Mr = -INFINITY, Lr = 0.f, O0 = 0.f, O1 = 0.f;
  constexpr int CB = 8;
  for (int cc = 0; cc < C; cc += CB) {
    float mv[CB], lv[CB], p0v[CB], p1v[CB];
#pragma unroll
    for (int t = 0; t < CB; ++t) {
      const bool in = cc + t < C;
      mv[t] = in ? ld_coh(mbase + 2 * (cc + t)) : -INFINITY;
      lv[t] = in ? ld_coh(mbase + 2 * (cc + t) + 1) : 0.f;
      p0v[t] = in ? ld_coh(pbase + (size_t)(cc + t) * hd) : 0.f;
      p1v[t] = in ? ld_coh(pbase + (size_t)(cc + t) * hd + 1) : 0.f;
    }
#pragma unroll
    for (int t = 0; t < CB; ++t) {
      if (mv[t] == -INFINITY) continue;
      const float Mn = fmaxf(Mr, mv[t]);
      const float a = Mr == -INFINITY ? 0.f : expf(Mr - Mn);
      const float bs = expf(mv[t] - Mn);
      O0 = O0 * a + p0v[t] * bs;
      O1 = O1 * a + p1v[t] * bs;
      Lr = Lr * a + lv[t] * bs;
      Mr = Mn;
    }
  }
  if (act) {
    if constexpr (MB == 1) {
      st_coh(P.att_o + o_at + dd, O0 / Lr);
      st_coh(P.att_o + o_at + dd + 1, O1 / Lr);
    } else {
      st_coh(P.att_o16 + o_at + dd, __builtin_bit_cast(uint16_t, (_Float16)(O0 / Lr)));
      st_coh(P.att_o16 + o_at + dd + 1, __builtin_bit_cast(uint16_t, (_Float16)(O1 / Lr)));
    }
  }
}

// Passes of a register group in attend_chunk: each pass gives every lane one
// 16-byte piece of a K row and of a V row (hd / 8 lanes per position).
constexpr int kAttnPasses = 8;

// Online-softmax partial of one (column, head) over positions [j0, j1): the
// running max M, the sum of exp Lsum and the unnormalised sum acc of exp * V
// (dims 8 sub .. 8 sub + 7, summed over the wave's position groups).  The
// first group's loads of rows before pos go out before `wait` runs (once,
// `waited` records it); rows from pos on were written in this step and are
// read after it.  False if the wait reported a failed barrier.
template <int HD, int MB, class Wait>
__device__ __forceinline__ bool attend_chunk(const Params& P, rsrc_t rk, rsrc_t rv, rsrc_t rq, int j0, int j1, int pos,
                                             bool& waited, Wait&& wait, float& M, float& Lsum, float (&acc)[8]) {
  constexpr int LP = HD / 8, PPW = 64 / LP;
  constexpr int NPASS = kAttnPasses;
  constexpr int GRP = PPW * NPASS;       // positions per register group
  const int lane = threadIdx.x & 63;
  const int sub = lane % LP, pidx = lane / LP;
  f32x4 qa = {0.f, 0.f, 0.f, 0.f}, qb = {0.f, 0.f, 0.f, 0.f};
  bool failed = false;
  for (int g0 = j0; g0 < j1; g0 += GRP) {
    u32x4 kr[NPASS], vr[NPASS];
    const bool pre = !waited;   // loads issued before the barrier skip the row at pos
#pragma unroll
    for (int t = 0; t < NPASS; ++t) {
      const int j = g0 + t * PPW + pidx;
      const uint32_t off = (j < j1 && (!pre || j < pos)) ? (uint32_t)(j * HD + 8 * sub) * 2u : kOOB;
      kr[t] = ld_kv(rk, off);
      vr[t] = ld_kv(rv, off);
    }
    if (pre) {
      waited = true;
      // no early return with this group's loads in flight: on the path out,
      // the compiler would have to assume them pending in the weight loop and
      // guard its registers with a full vmcnt(0) wait in every group
      if (!wait()) failed = true;
      if (g0 + GRP > pos) {
        // rows of this step's positions, written before the barrier
#pragma unroll
        for (int t = 0; t < NPASS; ++t) {
          const int j = g0 + t * PPW + pidx;
          if (j >= pos && j < j1) {
            const uint32_t off = (uint32_t)(j * HD + 8 * sub) * 2u;
            kr[t] = ld_kv(rk, off);
            vr[t] = ld_kv(rv, off);
          }
        }
      }
    }
    if (g0 == j0) {
      qa = ld_coh4(rq, (uint32_t)(32 * sub));
      qb = ld_coh4(rq, (uint32_t)(32 * sub + 16));
    }
    float s[NPASS];
    float mloc = -INFINITY;
#pragma unroll
    for (int t = 0; t < NPASS; ++t) {
      const int j = g0 + t * PPW + pidx;
      float dsum = dot8(kr[t], qa, qb, 0.f);
      dsum = group_sum<LP>(dsum);
      s[t] = j < j1 ? dsum : -INFINITY;
      mloc = fmaxf(mloc, s[t]);
    }
    const float Mn = fmaxf(M, wave_max(mloc));
    const float alpha = M == -INFINITY ? 0.f : expf(M - Mn);
    float lloc = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] *= alpha;
#pragma unroll
    for (int t = 0; t < NPASS; ++t) {
      const int j = g0 + t * PPW + pidx;
      const float e = j < j1 ? expf(s[t] - Mn) : 0.f;
      lloc += e;
      const f16x8 v = __builtin_bit_cast(f16x8, vr[t]);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(e, (float)v[q], acc[q]);
    }
    // every lane of a position group holds the same e: count it once
    Lsum = Lsum * alpha + wave_sum(sub == 0 ? lloc : 0.f);
    M = Mn;
  }
  // sum over the position groups of the wave: lanes sub, sub+LP, ...
#pragma unroll
  for (int q = 0; q < 8; ++q)
    for (int off = LP; off < 64; off <<= 1) acc[q] += __shfl_xor(acc[q], off, 64);
  return !failed;
}

// Attention by workgroups (the handle guarantees no more (column, head)
// pairs HB than workgroups).  Pair hb gets W workgroups: workgroup g < HB * W takes
// pair g / W, and its eight waves take chunks 8 (g mod W) .. 8 (g mod W) + 7
// of the pair's C = 8 W chunks.  The waves' partials meet in LDS and wave 0
// merges them after S1.  With W == 1 that is o.  Otherwise the workgroup's
// partial goes to memory and the last of the pair's W workgroups (arrival
// counter) merges the W partials.
//
// A wave reads its positions in register groups (attend_chunk: 32
// positions at head dim 128), and the attention phase lasts about as many
// group times as the busiest wave has groups; a split over W > 1 workgroups
// adds a merge through memory that costs about one group.  So: one
// workgroup (at most two groups per wave) up to 16 groups of positions,
// beyond that enough workgroups for one group per wave, but at most
// kMaxWgPerHead: at long contexts the K/V stream is bound by HBM, and more
// workgroups only add merge work and take workgroups from the GU cache
// warm-up.
constexpr int kMaxWgPerHead = 8;
__device__ __forceinline__ int wg_per_head(const Params& P, int pos) {
  const int HB = P.B * P.H, G = gridDim.x;   // HB <= G (checked when the handle is made)
  const int ctx_max = col_pos(P, pos, P.B - 1) + 1;
  const int per_wg = kWaves * (512 / P.hd) * kAttnPasses;   // positions of one group on every wave
  const int want = ctx_max <= 2 * per_wg ? 1 : min((ctx_max + per_wg - 1) / per_wg, kMaxWgPerHead);
  return max(1, min(min(want, G / HB), kChunkCap));
}

template <int HD, int MB, class Wait>
__device__ __forceinline__ bool attention_wg(const Params& P, int l, int pos, int pos_end, int wave, int W, Wait&& wait,
                                             float* part) {
  constexpr int LP = HD / 8;
  const int lane = threadIdx.x & 63, sub = lane % LP, pidx = lane / LP;
  const int H = P.H, HB = P.B * P.H, hb = blockIdx.x / W, k = blockIdx.x - hb * W;
  bool live = hb < HB;
  const int seq = live ? hb / H : 0, h = hb - seq * H, cpos = col_pos(P, pos, seq);
  live = live && cpos < pos_end;
  bool waited = false;
  float M = -INFINITY, Lsum = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (live) {
    const int ctx_max = col_pos(P, pos, P.B - 1) + 1, C = kWaves * W, CH = (ctx_max + C - 1) / C;
    const int c = k * kWaves + wave;
    const int j0 = min(cpos + 1, c * CH), j1 = min(cpos + 1, j0 + CH);
    const size_t head_elems = (size_t)P.max_ctx * HD;
    const int KH = kv_heads(P), kh = kv_seq(P, seq) * H + h;
    const rsrc_t rk = make_rsrc(P.kv + ((size_t)(l * 2 + 0) * KH + kh) * head_elems, (uint32_t)(head_elems * 2));
    const rsrc_t rv = make_rsrc(P.kv + ((size_t)(l * 2 + 1) * KH + kh) * head_elems, (uint32_t)(head_elems * 2));
    const rsrc_t rq = make_rsrc(P.qkv + (size_t)seq * 3 * P.q + h * HD, (uint32_t)(HD * 4));
    if (!attend_chunk<HD, MB>(P, rk, rv, rq, j0, j1, pos, waited, wait, M, Lsum, acc)) return false;
  }
  if (!waited && !wait()) return false;
  if (live) {
    float* pl = part + wave * (HD + 2);
    if (pidx == 0) {
#pragma unroll
      for (int q = 0; q < 8; ++q) pl[8 * sub + q] = acc[q];
    }
    if (lane == 0) { pl[HD] = M; pl[HD + 1] = Lsum; }
  }
  return true;
}


// Wave 0, after S1: the workgroup's pair from its eight waves' partials, in
// wave order (lane k owns dims 2k, 2k+1); then o, or the workgroup's partial
// and, for the pair's last workgroup, the merge of all W.
template <int MB>
__device__ __forceinline__ void w0_merge_wg(const Params& P, int pos, int pos_end, int W, const float* part) {
  const int lane = threadIdx.x & 63, hd = P.hd, H = P.H, HB = P.B * P.H;
  const int hb = blockIdx.x / W, k = blockIdx.x - hb * W;
  if (hb >= HB) return;
  const int seq = hb / H, h = hb - seq * H;
  if (col_pos(P, pos, seq) >= pos_end) return;
  const bool act = 2 * lane < hd;
  const int dd = act ? 2 * lane : 0;
  float Mx = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) Mx = fmaxf(Mx, part[w * (hd + 2) + hd]);
  float O0 = 0.f, O1 = 0.f, L = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float* pl = part + w * (hd + 2);
    const float m = pl[hd];
    if (m == -INFINITY) continue;   // a wave with no positions
    const float e = expf(m - Mx);
    O0 = __builtin_fmaf(e, pl[dd], O0);
    O1 = __builtin_fmaf(e, pl[dd + 1], O1);
    L = __builtin_fmaf(e, pl[hd + 1], L);
  }
  const size_t o_at = (size_t)seq * P.q + h * hd;
  if (W == 1) {
    if (act) {
      if constexpr (MB == 1) {
        st_coh(P.att_o + o_at + dd, O0 / L);
        st_coh(P.att_o + o_at + dd + 1, O1 / L);
      } else {
        st_coh(P.att_o16 + o_at + dd, __builtin_bit_cast(uint16_t, (_Float16)(O0 / L)));
        st_coh(P.att_o16 + o_at + dd + 1, __builtin_bit_cast(uint16_t, (_Float16)(O1 / L)));
      }
    }
    return;
  }
  float* pp = P.part + ((size_t)hb * P.max_chunks + k) * hd;
  float* pm = P.pml + ((size_t)hb * P.max_chunks + k) * 2;
  if (act) { st_coh(pp + dd, O0); st_coh(pp + dd + 1, O1); }
  if (lane == 0) { st_coh(pm, Mx); st_coh(pm + 1, L); }
  wait_vm0();   // the partial is visible before the workgroup counts itself
  uint32_t old = 0;
  if (lane == 0) old = atomic_add_coh(P.ctl + kCtlHead0 + hb, 1u);
  old = (uint32_t)__builtin_amdgcn_readlane((int)old, 0);
  if (old == (uint32_t)(W - 1)) merge_head<MB>(P, hb, W, o_at);
}

// ---------------------------------------------------------------------------
// wave 0: phase outputs
// ---------------------------------------------------------------------------
// out holds the phase's row sums, row-major over sequences: out[row * MB + b].
// scl[b] is sequence b's norm scale for the phase (1 where there is no norm).
// QKV rows come in pairs (2i, 2i+1) of one head, which are exactly the pairs
// the rotary embedding rotates: q is rotated, scaled by 1/sqrt(hd) and
// stored for attention; k is rotated and v taken as it is, both rounded to
// fp16 and appended to the KV cache at (layer l, position pos).
template <int MB, bool MOE = false>
__device__ __forceinline__ void w0_store_outputs(const Params& P, int ph, int l, int pos, int pos_end,
                                                 const int* tab_wg, int lg_mode, const float* scl,
                                                 const float* out, float* xown, const float* rope_lds,
                                                 const float* gs_next, const uint16_t* moe_wr = nullptr,
                                                 bool store_x = true) {
  const int lane = threadIdx.x & 63, B = P.B;
  if (!is_gemv(ph)) return;
  if (MOE && ph == PH_GU) {
    // mixture of experts: this workgroup's row pairs j of its slot's expert
    // e, silu(gate) * up with the row scales, times the expert's routing
    // weight, into the slot's part of the hidden vector
    const int slot = rfl(tab_wg[kTabMoeSlot]), q0 = rfl(tab_wg[kTabMoeSlot + 1]), nq = rfl(tab_wg[kTabMoeSlot + 2]) - q0;
    // the routing wave 0 kept in LDS (aux, which rope_lds points at)
    const int e = reinterpret_cast<const int*>(rope_lds)[kAuxRoute + slot];
    const float w = rope_lds[kAuxRoute + kMoeMaxTopK + slot];
    const float* sc = P.esc + (size_t)l * P.sc_stride + (size_t)2 * ((size_t)e * P.Fe + q0);
    for (int t = lane; t < nq; t += 64) {
      // (MXFP4 rows have no row scale: their block scales were applied in the dot)
      const float gt = out[kMoeOutPairs + 2 * t] * scl[0] * (P.mx ? 1.0f : ldg(sc + 2 * t));
      const float up = out[kMoeOutPairs + 2 * t + 1] * scl[0] * (P.mx ? 1.0f : ldg(sc + 2 * t + 1));
      st_coh(P.act + (size_t)slot * P.Fe + q0 + t, gt / (1.0f + expf(-gt)) * up * w);
    }
    return;
  }
  const int p0 = rfl(tab_wg[2 * ph]);
  const int n = rfl(tab_wg[2 * ph + 1]) - p0;
  const int own = kOwnFloats / MB;
  if (ph == PH_QKV) {
    wait_vm0();   // rope_lds: the step's rotary rows (LDS DMA during the QKV GEMV)
    const int q = P.q, hd = P.hd, KH = kv_heads(P);
    const float qscale = 1.0f / sqrtf((float)hd);
    const size_t head_elems = (size_t)P.max_ctx * hd;
    for (int e = lane; e < n * MB; e += 64) {
      const int t = e / MB, b = e - t * MB;
      const int cpos = col_pos(P, pos, b);
      if (b < B && cpos < pos_end) {
        const int r = 2 * (p0 + t);                       // even row of Wqkv
        const size_t kvrow = (size_t)(kv_seq(P, b) * P.H) * head_elems + (size_t)cpos * hd;
        const int part = r / q, rr = r - part * q;        // 0: q, 1: k, 2: v
        const int h = rr / hd, i = (rr - h * hd) >> 1;
        const float y0 = out[2 * t * MB + b] * scl[b], y1 = out[(2 * t + 1) * MB + b] * scl[b];
        if (part == 2) {
          const uint32_t vb = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)y0) |
                              ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)y1) << 16);
          uint16_t* vc = P.kv + ((size_t)(l * 2 + 1) * KH + h) * head_elems + kvrow + 2 * i;
          st_coh(reinterpret_cast<uint32_t*>(vc), vb);
        } else {
          const float cs = rope_lds[(cpos - pos) * hd + 2 * i];
          const float sn = rope_lds[(cpos - pos) * hd + 2 * i + 1];
          const float z0 = y0 * cs - y1 * sn, z1 = y0 * sn + y1 * cs;
          if (part == 0) {
            st_coh(P.qkv + (size_t)b * 3 * q + rr, z0 * qscale);
            st_coh(P.qkv + (size_t)b * 3 * q + rr + 1, z1 * qscale);
          } else {
            const uint32_t kb = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)z0) |
                                ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)z1) << 16);
            uint16_t* kc = P.kv + ((size_t)(l * 2) * KH + h) * head_elems + kvrow + 2 * i;
            st_coh(reinterpret_cast<uint32_t*>(kc), kb);
          }
        }
      }
    }
  } else if (ph == PH_O || ph == PH_DOWN) {
    float ss = 0.f;
    if constexpr (MB == 1) {
      for (int t = lane; t < 2 * n; t += 64) {
        const float v = xown[t] + out[t];
        xown[t] = v;
        st_coh(P.x + 2 * p0 + t, v);
      }
    } else {
      // batched: the next normed phase's input, x times its gains (held in
      // gs since that phase's gains were fetched), in fp16, and this
      // workgroup's share of sum(x^2).  Lane: sequence b = lane % 8, 8-row
      // blocks k = lane / 8, + 8, ... (the workgroup's 2n rows are a multiple
      // of 8), each one 16-byte store.  x itself is stored only when the
      // launch ends here (store_x): the next token starts from its embedding,
      // and within a launch only this workgroup reads its rows (xown).
      const int b = lane & (MB - 1);
      const rsrc_t rx = make_rsrc(P.x, (uint32_t)(B * P.d * 4));
      const rsrc_t rg = make_rsrc(P.xg16, (uint32_t)(kMaxBatch * P.d * 2));
      for (int k = lane >> 3; k < (2 * n) >> 3; k += 8) {
        if (b < B) {
          float v[8];
          f16x8 h;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int t = 8 * k + i;
            v[i] = xown[b * own + t] + out[t * MB + b];
            xown[b * own + t] = v[i];
            h[i] = (_Float16)(v[i] * gs_next[2 * p0 + t]);
            ss += v[i] * v[i];
          }
          const int r = 2 * p0 + 8 * k;
          st_coh16(rg, (uint32_t)(blk8(b, r) * 2), __builtin_bit_cast(u32x4, h));
          if (store_x) {
            st_coh16(rx, (uint32_t)(((size_t)b * P.d + r) * 4), __builtin_bit_cast(u32x4, f32x4{v[0], v[1], v[2], v[3]}));
            st_coh16(rx, (uint32_t)(((size_t)b * P.d + r + 4) * 4), __builtin_bit_cast(u32x4, f32x4{v[4], v[5], v[6], v[7]}));
          }
        }
      }
    }
    if (MOE && ph == PH_O && lane < P.E) {
      // mixture of experts: this workgroup's share of each router logit,
      // sum over its rows r of router[e][r] * g[r] * x[r] (g: the FFN norm's
      // gains, in gs since the QKV phase fetched them; the router columns
      // staged in the O phase)
      float acc = 0.f;
      const _Float16* wr = reinterpret_cast<const _Float16*>(moe_wr) + lane * 2 * n;
      for (int t = 0; t < 2 * n; ++t) acc = __builtin_fmaf((float)wr[t], gs_next[2 * p0 + t] * xown[t], acc);
      st_coh(P.rpart + (size_t)blockIdx.x * kMoeMaxExperts + lane, acc);
    }
    if constexpr (MB > 1) {
      // lane l holds sequence l % MB's share (64 is a multiple of MB)
      ss += __shfl_xor(ss, 8, 64);
      ss += __shfl_xor(ss, 16, 64);
      ss += __shfl_xor(ss, 32, 64);
      if (lane < MB) st_coh(P.ssp + (size_t)blockIdx.x * kMaxBatch + lane, ss);
    }
  } else if (ph == PH_GU && MB > 1) {
    // batched: lane: sequence b = lane % 8, outputs 8k .. 8k + 7 for blocks
    // k = lane / 8, + 8, ... (n is a multiple of 8), one 16-byte store each
    const int b = lane & (MB - 1);
    const rsrc_t ra = make_rsrc(P.act16, (uint32_t)(kMaxBatch * P.F * 2));
    for (int k = lane >> 3; k < n >> 3; k += 8) {
      if (b < B) {
        f16x8 h;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int t = 8 * k + i;
          const float gt = out[2 * t * MB + b] * scl[b], up = out[(2 * t + 1) * MB + b] * scl[b];
          h[i] = (_Float16)(gt / (1.0f + expf(-gt)) * up);
        }
        st_coh16(ra, (uint32_t)(blk8(b, p0 + 8 * k) * 2), __builtin_bit_cast(u32x4, h));
      }
    }
  } else if (ph == PH_GU) {
    for (int e = lane; e < n * MB; e += 64) {
      const int t = e / MB, b = e - t * MB;
      if (b < B) {
        const float gt = out[2 * t * MB + b] * scl[b], up = out[(2 * t + 1) * MB + b] * scl[b];
        const float a = gt / (1.0f + expf(-gt)) * up;
        st_coh(P.act + p0 + t, a);
      }
    }
  } else if (ph == PH_LM && MB == 1) {
    // this workgroup's best logit (lowest row on ties)
    float best = -INFINITY;
    int bidx = 0x7fffffff;
    for (int t = lane; t < 2 * n; t += 64) {
      const float v = out[t] * scl[0];
      if (v > best) { best = v; bidx = 2 * p0 + t; }
      // logits: 1 = the device buffer; 2 = the host's pinned buffer (a server
      // launch keeps running while the host reads them)
      if (lg_mode == 1) st_g(P.logits + 2 * p0 + t, v);
      else if (lg_mode == 2) st_sys(P.lg_sys + 2 * p0 + t, v);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(best, off, 64);
      const int oi = __shfl_xor(bidx, off, 64);
      if (ov > best || (ov == best && oi < bidx)) { best = ov; bidx = oi; }
    }
    if (lane == 0) {
      st_coh(P.amax_v + blockIdx.x, best);
      st_coh(P.amax_i + blockIdx.x, bidx);
    }
  } else if (ph == PH_LM) {
    // batched: lane l scans sequence b = l % MB over rows l / MB, l / MB + 8,
    // ... (consecutive LDS words across the wave), so each sequence's best
    // is reduced over its 8 lanes only; partials go to [workgroup][kMaxBatch]
    const int b = lane & (MB - 1);
    float best = -INFINITY;
    int bidx = 0x7fffffff;
    if (b < B) {
      const float sb = scl[b];
      for (int t = lane / MB; t < 2 * n; t += 64 / MB) {
        const float v = out[t * MB + b] * sb;
        if (v > best) { best = v; bidx = 2 * p0 + t; }
        if (lg_mode == 1) st_g(P.logits + (size_t)b * P.Vlm + 2 * p0 + t, v);
        else if (lg_mode == 2) st_sys(P.lg_sys + (size_t)b * P.Vlm + 2 * p0 + t, v);
      }
    }
#pragma unroll
    for (int off = MB; off < 64; off <<= 1) {
      const float ov = __shfl_xor(best, off, 64);
      const int oi = __shfl_xor(bidx, off, 64);
      if (ov > best || (ov == best && oi < bidx)) { best = ov; bidx = oi; }
    }
    if (lane < B) {
      st_coh(P.amax_v + (size_t)blockIdx.x * kMaxBatch + lane, best);
      st_coh(P.amax_i + (size_t)blockIdx.x * kMaxBatch + lane, bidx);
    }
  }
}

// Greedy token of every sequence = argmax over the workgroups' partials
// (lowest index on ties).  Every workgroup computes it (it is the next
// token's input); workgroup 0 publishes it.  All sequences' partials are
// requested before any is reduced.
template <int MB>
__device__ __forceinline__ void w0_argmax(const Params& P, int i, int cur_col, int* tok) {
  const int lane = threadIdx.x & 63, G = gridDim.x, B = P.B;
  auto better = [](float v, int ix, float bv, int bi) { return v > bv || (v == bv && ix < bi); };
  if constexpr (MB == 1) {
    const rsrc_t rv = make_rsrc(P.amax_v, (uint32_t)(G * 4)), ri = make_rsrc(P.amax_i, (uint32_t)(G * 4));
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    constexpr int K = 4;   // partials per lane per pass, all requested before any is compared
    for (int t0 = 0; t0 < G; t0 += 64 * K) {
      float v[K];
      int ix[K];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int t = t0 + lane + 64 * k;
        const uint32_t off = t < G ? (uint32_t)t * 4u : kOOB;
        v[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rv, off, 0, kAuxSc1));
        ix[k] = (int)__builtin_amdgcn_raw_buffer_load_b32(ri, off, 0, kAuxSc1);
      }
#pragma unroll
      for (int k = 0; k < K; ++k)
        if (t0 + lane + 64 * k < G && better(v[k], ix[k], bv, bi)) { bv = v[k]; bi = ix[k]; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    tok[0] = (bi == 0x7fffffff) ? 0 : bi;
  } else {
    // partials at [workgroup][kMaxBatch]: lane l takes sequence l % MB of
    // workgroups l / MB + 8 j (consecutive words across the wave), all
    // requested before any is compared, then the 8 lanes of each sequence
    // combine theirs
    const int b = lane & (MB - 1);
    const uint32_t bytes = (uint32_t)(G * kMaxBatch * 4);
    const rsrc_t rv = make_rsrc(P.amax_v, bytes), ri = make_rsrc(P.amax_i, bytes);
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    constexpr int J = 32;
    for (int g0 = 0; g0 < G; g0 += J * (64 / MB)) {
      float v[J];
      int ix[J];
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int g = g0 + lane / MB + (64 / MB) * j;
        const uint32_t off = (b < B && g < G) ? (uint32_t)(g * kMaxBatch + b) * 4u : kOOB;
        v[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rv, off, 0, kAuxSc1));
        ix[j] = (int)__builtin_amdgcn_raw_buffer_load_b32(ri, off, 0, kAuxSc1);
      }
#pragma unroll
      for (int j = 0; j < J; ++j)
        if (b < B && g0 + lane / MB + (64 / MB) * j < G && better(v[j], ix[j], bv, bi)) { bv = v[j]; bi = ix[j]; }
    }
#pragma unroll
    for (int off = MB; off < 64; off <<= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
#pragma unroll
    for (int bb = 0; bb < MB; ++bb) {
      const int t = __builtin_amdgcn_readlane(bi, bb);
      tok[bb] = (t == 0x7fffffff) ? 0 : t;
    }
  }
#pragma unroll
  for (int b = 0; b < MB; ++b) {
    if (b < B && blockIdx.x == 0 && lane == 0) {
      if (cur_col < 0) st_coh(P.tok_cur + b, tok[b]);
      else if (b == cur_col) st_coh(P.tok_cur, tok[b]);
      st_coh(P.tok_out + (size_t)i * P.B + b, tok[b]);
    }
  }
}

// ---------------------------------------------------------------------------
// decode server requests (wave 0)
// ---------------------------------------------------------------------------
// A request as wave 0 holds it: state 1 = request k is posted (flags and
// input tokens below), -1 = the launch ends at k, 0 = not known yet.
struct Request { int state; int flags; int tok[kMaxBatch]; };

__device__ __forceinline__ uint64_t srv_tag(const Launch& A, uint32_t k, bool end) {
  return ((uint64_t)A.srv_epoch << 32) | (uint64_t)((k + 1u) | (end ? kMailClosed : 0u));
}

__device__ __forceinline__ void take_fields(int v, Request& rq) {
  rq.flags = __builtin_amdgcn_readlane(v, 0);
#pragma unroll
  for (int b = 0; b < kMaxBatch; ++b) rq.tok[b] = __builtin_amdgcn_readlane(v, 1 + b);
}

// Workgroup 0: request k from the host mailbox.  A posted request (ctl counts
// past k) has its fields in place: the host writes them before it raises
// ctl, and the field loads issue only after the ctl load has returned.  The
// request, or the end, is copied to every device slot, fields before tag.
// With `block`, waits up to the idle bound, then closes the mailbox at k by
// compare-and-swap; the value that swap leaves (the host's post or the
// close) decides.  Without `block`, returns 0 when nothing is decided yet.
__device__ int w0_host_request(const Params& P, const Launch& A, uint32_t k, bool block, Request& rq) {
  const int lane = threadIdx.x & 63;
  Mailbox* m = P.mail;
  const uint64_t t0 = wall_clock64();
  int state;
  while (true) {
    const uint32_t c = (uint32_t)rfl((int)ld_sys(&m->ctl));
    if ((c & ~kMailClosed) > k) { state = 1; break; }
    if (c & kMailClosed) { state = -1; break; }
    if (!block) return 0;
    const uint64_t waited = wall_clock64() - t0;
    if (waited > (uint64_t)A.idle_ticks + (uint64_t)P.watchdog_ticks) {
      // the close did not take (host memory without device atomics): end
      // with the timeout error rather than spin
      if (lane == 0) {
        uint32_t expected = 0u;
        __hip_atomic_compare_exchange_strong((guint*)(P.ctl + kCtlErr), &expected, (uint32_t)kDevErrTimeout,
                                             __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      state = -1;
      break;
    }
    if (waited > (uint64_t)A.idle_ticks) {
      if (lane == 0) {
        uint32_t expected = c;
        __hip_atomic_compare_exchange_strong((guint*)&m->ctl, &expected, c | kMailClosed, __ATOMIC_RELAXED,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      }
      wait_vm0();
      continue;
    }
    __builtin_amdgcn_s_sleep(4);
  }
  const int slot = (int)(k % kMailRing) * kReqWords;
  if (state > 0) {
    const int v = lane <= kMaxBatch ? ld_sys(&m->req[0][0] + slot + lane) : 0;
    take_fields(v, rq);
    if (lane <= kMaxBatch)
      for (int c = 0; c < kSrvCopies; ++c) st_coh(P.srv_slot + c * kMailRing * kReqWords + slot + 2 + lane, v);
  }
  wait_vm0();   // the fields have landed before any tag
  if (lane < kSrvCopies)
    st_coh64(reinterpret_cast<uint64_t*>(P.srv_slot + lane * kMailRing * kReqWords + slot), srv_tag(A, k, state < 0));
  rq.state = state;
  return state;
}

// Every other workgroup: request k from its device slot copy (tag first, then
// the fields, which workgroup 0 stored before the tag).  With `block`, waits
// until workgroup 0 has decided; that takes at most the idle bound, so a wait
// past it plus the watchdog bound, or an error raised by any workgroup, ends
// the launch here (the watchdog case raising the timeout error).
__device__ int w0_device_request(const Params& P, const Launch& A, uint32_t k, bool block, Request& rq) {
  const int lane = threadIdx.x & 63;
  const int32_t* slot = P.srv_slot + (blockIdx.x % kSrvCopies) * kMailRing * kReqWords + (k % kMailRing) * kReqWords;
  const uint64_t go = srv_tag(A, k, false), end = srv_tag(A, k, true);
  const uint64_t t0 = wall_clock64();
  const uint64_t limit = (uint64_t)A.idle_ticks + (uint64_t)P.watchdog_ticks;
  int state;
  while (true) {
    const uint64_t t = ld_coh64(reinterpret_cast<const uint64_t*>(slot));
    const uint64_t tu = ((uint64_t)(uint32_t)rfl((int)(t >> 32)) << 32) | (uint32_t)rfl((int)(uint32_t)t);
    if (tu == go) { state = 1; break; }
    if (tu == end) { state = -1; break; }
    if (!block) return 0;
    if (rfl((int)ld_coh(P.ctl + kCtlErr)) != 0) { state = -1; break; }
    if (wall_clock64() - t0 > limit) {
      if (lane == 0) {
        uint32_t expected = 0u;
        __hip_atomic_compare_exchange_strong((guint*)(P.ctl + kCtlErr), &expected, (uint32_t)kDevErrTimeout,
                                             __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      state = -1;
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  if (state > 0) take_fields(lane <= kMaxBatch ? ld_coh(slot + 2 + lane) : 0, rq);
  rq.state = state;
  return state;
}

__device__ __forceinline__ int srv_request(const Params& P, const Launch& A, uint32_t k, bool block, Request& rq) {
  return blockIdx.x == 0 ? w0_host_request(P, A, k, block, rq) : w0_device_request(P, A, k, block, rq);
}

// Workgroup 0 after request k's greedy tokens: store them for the host now;
// the completion count follows once they have landed (srv_flush_done), at
// this wave's next wait for its stores or before it blocks for a request.
template <int MB>
__device__ __forceinline__ void srv_post_tokens(const Params& P, uint32_t k, const int* tok, int& done_pending) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int b = 0; b < MB; ++b)
    if (lane == b && b < P.B) st_sys(&P.mail->tok[k % kMailRing][b], tok[b]);
  done_pending = (int)k + 1;
}
__device__ __forceinline__ void srv_flush_done(const Params& P, int& done_pending) {
  if (done_pending <= 0) return;
  wait_vm0();
  if ((threadIdx.x & 63) == 0) st_sys(&P.mail->done, (uint32_t)done_pending);
  done_pending = 0;
}

// where the LM head's logits go for token i: none, the device buffer (the
// last token of a launch that wants them) or the host (a server request
// that wants them)
__device__ __forceinline__ int lg_mode(const Launch& A, int i, bool cur_lg) {
  if (DEC_COLD(A.server)) return cur_lg ? 2 : 0;
  return A.write_logits && i == A.n_tok - 1 ? 1 : 0;
}

// ---------------------------------------------------------------------------
// the resident kernel
// ---------------------------------------------------------------------------
// Both roles walk the same phase sequence and meet at the same workgroup
// barriers: S1a (raw phase input in LDS; wave 0 has passed the grid
// barrier), S1 (input ready: gains applied or attention merged) and S2
// (phase outputs in LDS).

// A streamer's attention phase: its units (the first one's cached rows are
// requested before S1a), then S1 and S2 as in every phase.  False if wave 0
// reported a failed grid barrier.
// Cache warm-up in the attention gap: a streamer of a workgroup without a
// head requests the first GU row pair of its share (10 KB) with ordinary,
// cache-allocating loads into an LDS sink.  HBM is otherwise idle while the
// heads' workgroups compute attention, and the GU phase's own streaming loads
// of those blocks then hit the device-side cache.  A streamer takes no more
// than one row pair: it issued its O-phase weight loads before these, and
// its first O-phase wait (in issue order) would also wait for them.
__device__ __forceinline__ void warm_gu(const Params& P, const int* tab, int l, float* sink) {
  const int lane = threadIdx.x & 63;
  const int* e = tab + PH_GU * kTabStride;
  if (rfl(e[T_LEFT]) <= 0) return;
  const rsrc_t r = make_rsrc(gemv_base(P, PH_GU, rfl(l)), (uint32_t)rfl(e[T_NBYTES]));
  const uint32_t off = (uint32_t)rfl(e[T_OFF]), rowb = (uint32_t)rfl(e[T_ROWB]);
  for (uint32_t k = 0; k < 2 * rowb / 1024u; ++k) dma16_ld(r, sink, off + 1024u * k + 16u * lane);
}

// Wave 0 of such a workgroup, once it has arrived at the barrier before O,
// warms more: for each streamer, the GU blocks just past the row pair the
// streamer warms itself, up to kW0WarmBlocks of 1 KB, within the streamer's
// share.  Wave 0 has nothing else in flight there, but its first poll for the
// O release waits behind these loads, so they must land within the attention
// window.  12 blocks per streamer measured best over positions 128-639 at
// d 2560 with 63 barrier groups: 24 held the O release back by about 3 us,
// 8 and 10 warmed too little.  With the streamers' own row pair that warms
// about 33 MB of GU rows per layer over the 236 workgroups without a head,
// close to the 32 MB of L2, so few warmed rows are evicted and fetched again.
constexpr int kW0WarmBlocks = 12;
__device__ __forceinline__ void w0_warm_gu(const Params& P, const int* tab_all, int l, float* sink) {
  const int lane = threadIdx.x & 63;
  const int* e0 = tab_all + PH_GU * kTabStride;
  const rsrc_t r = make_rsrc(gemv_base(P, PH_GU, rfl(l)), (uint32_t)rfl(e0[T_NBYTES]));
  for (int s = 0; s < kStreamers; ++s) {
    const int* e = tab_all + s * kStreamerTab + PH_GU * kTabStride;
    const uint32_t left = (uint32_t)max(rfl(e[T_LEFT]), 0);
    const uint32_t off = (uint32_t)rfl(e[T_OFF]), rowb = (uint32_t)rfl(e[T_ROWB]);
    const uint32_t end = off + 2048u * left;   // the streamer's units are about 2 KB each
    for (uint32_t k = 0; k < (uint32_t)kW0WarmBlocks; ++k) {
      const uint32_t b = off + 2u * rowb + 1024u * k;
      if (b + 1024u <= end) dma16_ld(r, sink, b + 16u * lane);
    }
  }
}

// The same for the batched kernel (workgroups past the B*H attention pairs):
// the 1 KB GU tiles past each streamer's first group (in its registers),
// up to kW0WarmTiles per streamer.  At batch 8, with these workgroups
// holding the extra gate/up group (split_tail): 16, 24, 32, 40 and 48 tiles
// gave 1.471, 1.452, 1.458, 1.519 and 1.540 ms per step.
constexpr int kW0WarmTiles = 24;
__device__ __forceinline__ void w0_warm_tiles(const Params& P, const int* tab_all, int l, float* sink) {
  const int lane = threadIdx.x & 63;
  const int* e0 = tab_all + PH_GU * kTabStride;
  const rsrc_t r = make_rsrc(gemv_base(P, PH_GU, rfl(l)), (uint32_t)rfl(e0[T_NBYTES]));
  for (int s = 0; s < kStreamers; ++s) {
    const int* e = tab_all + s * kStreamerTab + PH_GU * kTabStride;
    const uint32_t left = (uint32_t)max(rfl(e[T_LEFT]), 0);
    const uint32_t off = (uint32_t)rfl(e[T_OFF]);
    const uint32_t end = off + 1024u * left;
    for (uint32_t k = 0; k < (uint32_t)kW0WarmTiles; ++k) {
      const uint32_t b = off + 1024u * (kTilesInFlight + k);
      if (b + 1024u <= end) dma16_ld(r, sink, b + 16u * lane);
    }
  }
}

template <int MB, int HD>
__device__ __forceinline__ bool streamer_attention(const Params& P, const Launch& A, const PhaseIt& id, const int* si,
                                                   float* aux, const int* tab = nullptr, float* sink = nullptr) {
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  auto wait_s = [&]() {
    __syncthreads();   // S1a
    return si[12] != 0;
  };
  const int pos = step_pos(P, A, id.i);
  // (not with few heads: their workgroups skip the QKV rows and the gap is short)
  if constexpr (MB == 1)
    if (P.E == 0 && P.H > (int)gridDim.x / 32 && (int)blockIdx.x / wg_per_head(P, pos) >= P.H)
      warm_gu(P, tab, id.l, sink);
  bool ok;
  ok = attention_wg<HD, MB>(P, id.l, pos, A.pos_end, wave, wg_per_head(P, pos), wait_s, aux + kAuxPart);
  if (DEC_COLD(!ok)) return false;
  wait_vm0();   // this wave's stores are complete before wave 0 arrives at the grid barrier
  __syncthreads();   // S1
  __syncthreads();   // S2
  return true;
}

// ---------------------------------------------------------------------------
// mixture of experts (batch 1)
// ---------------------------------------------------------------------------
// A layer's MLP is top_k of E SwiGLU experts whose rows are FP8 E4M3 codes
// with one fp32 scale each: at batch 1 only the chosen experts' bytes are
// read, which is what makes large mixture-of-experts models fast at batch 1
// (page 標準GPUによるリアルタイムLLM推論, section Hackerたちの意見; page
// 「ソフトウェア・ファースト」戦略でGPUの限界を突破…, section 今後のマイルストーンと課題).
// The GU phase's ordinary weight stream is the fp16 router [E, d], all of it
// in every workgroup, so its first blocks are prefetched across the barrier
// like any phase's.  Then every wave takes the top_k experts from the
// router's logits in LDS (moe_route), and the streamers read the chosen
// experts' rows (moe_stream): in GU the workgroups form top_k slots that
// split their expert's gate/up row pairs; in DOWN each workgroup keeps its
// dense share of the d output rows and reads, per row pair, the top_k
// experts' rows in turn.  Expert loads start once the routing is known, so
// they are not prefetched across the barrier.

// 16 E4M3 codes of each of two rows (one 16-byte load per row) times the
// same 16 fp32 inputs; fp32 accumulate.  The hardware conversion decodes
// OCP E4M3 exactly.
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void dot16_e4m3x2(u32x4 w0, u32x4 w1, const float* x, float& a0, float& a1) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 xv = *reinterpret_cast<const f32x4*>(x + 4 * i);
    const uint32_t c0 = w0[i], c1 = w1[i];
    const f32x2 l0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c0, false), h0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c0, true);
    const f32x2 l1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c1, false), h1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c1, true);
    const float x0 = xv[0], x1 = xv[1], x2 = xv[2], x3 = xv[3];
    a0 = __builtin_fmaf(l0[0], x0, a0);
    a0 = __builtin_fmaf(l0[1], x1, a0);
    a0 = __builtin_fmaf(h0[0], x2, a0);
    a0 = __builtin_fmaf(h0[1], x3, a0);
    a1 = __builtin_fmaf(l1[0], x0, a1);
    a1 = __builtin_fmaf(l1[1], x1, a1);
    a1 = __builtin_fmaf(h1[0], x2, a1);
    a1 = __builtin_fmaf(h1[1], x3, a1);
  }
}

// The router's logits are sums over the residual rows: every workgroup's O
// publication adds its own rows' share, router[e][r] * g[r] * x[r] for the
// FFN norm's gains g, into P.rpart[workgroup][e].  After the barrier each
// wave w sums the shares of workgroups w, w + 8, ... in that order
// (moe_router_issue / moe_router_finish, into LDS), and every wave adds the
// eight sums in wave order: the same bits in every wave and every workgroup.
// Split in two so that the shares' loads are in flight while the wave
// applies the norm gains: moe_router_issue requests the first 32 shares of
// this wave's workgroups (all of them for a grid of up to 256),
// moe_router_finish adds them (and any further ones) in workgroup order and
// stores the wave's sum.
constexpr int kRouterChunk = 32;
__device__ __forceinline__ void moe_router_issue(const Params& P, float (&v)[kRouterChunk]) {
  const int lane = threadIdx.x & 63, w = rfl((int)(threadIdx.x >> 6)), G = gridDim.x;
#pragma unroll
  for (int k = 0; k < kRouterChunk; ++k) {
    const int g = w + kWaves * k;
    v[k] = (lane < P.E && g < G) ? ld_coh(P.rpart + (size_t)g * kMoeMaxExperts + lane) : 0.f;
  }
}
__device__ __forceinline__ void moe_router_finish(const Params& P, const float (&v)[kRouterChunk], float* rs) {
  const int lane = threadIdx.x & 63, w = rfl((int)(threadIdx.x >> 6)), G = gridDim.x;
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < kRouterChunk; ++k) acc += v[k];
  if (lane < P.E)
    for (int g = w + kWaves * kRouterChunk; g < G; g += kWaves) acc += ld_coh(P.rpart + (size_t)g * kMoeMaxExperts + lane);
  rs[w * kMoeMaxExperts + lane] = acc;
}

// 32 MXFP4 weights of each of two rows (a 16-byte load per row: one block)
// times the same 32 fp32 inputs; fp32 accumulate.  v_cvt_scalef32_pk_f32_fp4
// turns one byte into its two E2M1 values (low nibble first) times the
// block's scale.
__device__ __forceinline__ float e8m0_float(uint32_t s) {
  // 2^(s - 127): the exponent field of an fp32, 2^-127 as a subnormal, 0xFF NaN
  return __builtin_bit_cast(float, s == 0u ? 0x00400000u : (s == 255u ? 0x7FC00000u : s << 23));
}
__device__ __forceinline__ void dot32_mxfp4x2(u32x4 w0, u32x4 w1, float s0, float s1, const float* x, float& a0,
                                              float& a1) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 xa = *reinterpret_cast<const f32x4*>(x + 8 * i);
    const f32x4 xb = *reinterpret_cast<const f32x4*>(x + 8 * i + 4);
    const uint32_t c0 = w0[i], c1 = w1[i];
    const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c0, s0, 0);
    const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c0, s0, 1);
    const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c0, s0, 2);
    const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c0, s0, 3);
    const f32x2 q0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c1, s1, 0);
    const f32x2 q1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c1, s1, 1);
    const f32x2 q2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c1, s1, 2);
    const f32x2 q3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c1, s1, 3);
    const float x0 = xa[0], x1 = xa[1], x2 = xa[2], x3 = xa[3], x4 = xb[0], x5 = xb[1], x6 = xb[2], x7 = xb[3];
    a0 = __builtin_fmaf(p0[0], x0, a0);
    a0 = __builtin_fmaf(p0[1], x1, a0);
    a0 = __builtin_fmaf(p1[0], x2, a0);
    a0 = __builtin_fmaf(p1[1], x3, a0);
    a0 = __builtin_fmaf(p2[0], x4, a0);
    a0 = __builtin_fmaf(p2[1], x5, a0);
    a0 = __builtin_fmaf(p3[0], x6, a0);
    a0 = __builtin_fmaf(p3[1], x7, a0);
    a1 = __builtin_fmaf(q0[0], x0, a1);
    a1 = __builtin_fmaf(q0[1], x1, a1);
    a1 = __builtin_fmaf(q1[0], x2, a1);
    a1 = __builtin_fmaf(q1[1], x3, a1);
    a1 = __builtin_fmaf(q2[0], x4, a1);
    a1 = __builtin_fmaf(q2[1], x5, a1);
    a1 = __builtin_fmaf(q3[0], x6, a1);
    a1 = __builtin_fmaf(q3[1], x7, a1);
  }
}

// Every wave, into its routing words rt (LDS, 16 per wave): the top_k
// experts of the router's logits (the sums rs of moe_router_finish, times the
// phase's norm scale, formed here from the waves' shares of sum(x^2) in the
// order wave 0 forms it) -- largest logit first, the lower index first on
// equal logits -- then from word 8 their weights, the softmax of the chosen
// logits.
__device__ __forceinline__ void moe_route(const Params& P, const float* rs, const float* red, float* rt) {
  const int lane = threadIdx.x & 63;
  float ss = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) ss += red[w];
  const float scale = 1.0f / sqrtf(ss / (float)P.d + P.eps);
  float sum = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) sum += rs[w * kMoeMaxExperts + lane];
  float v = lane < P.E ? sum * scale : -INFINITY;
  float mine = 0.f;   // lane s: the s-th chosen logit
  for (int s = 0; s < P.topk; ++s) {
    // the largest remaining logit (DPP maximum), at its lowest lane (ballot)
    const float best = wave_max(v);
    const uint64_t hit = __ballot(v == best);
    const int bi = min(hit ? (int)__builtin_ctzll(hit) : 0, P.E - 1);
    if (lane == s) {
      reinterpret_cast<int*>(rt)[s] = bi;
      mine = best;
    }
    if (lane == bi) v = -INFINITY;
  }
  const float top = readlane(mine, 0);
  const float ex = lane < P.topk ? expf(mine - top) : 0.f;
  const float den = wave_sum(ex);
  if (lane < P.topk) rt[kMoeMaxTopK + lane] = ex / den;
}

// LDS of the down phase's row scales: [slot][2 np] for the workgroup's np
// output row pairs (wave 0 fills it with the phase input; aux floats from
// kAuxMoe on, past the rotary rows and the attention partials)
constexpr int kAuxMoe = 1536;
static_assert(kAuxMoe + kMoeScaleFloats <= kAuxFloats, "aux LDS");

// Streamer s's share of a routed phase -- GU: gate/up row pairs [q0, q1) of
// the slot's expert; DOWN: every chosen expert's rows of the workgroup's
// output pairs.  A unit is a 1 KB piece of each of a row pair's two rows.
struct MoeGeo {
  int p0, np, npc, tail, nsl, per, u0, n;
};
template <bool DOWN, bool MX>
__device__ __forceinline__ MoeGeo moe_geo(const Params& P, int s, const int* tab_wg) {
  MoeGeo g;
  g.p0 = rfl(tab_wg[DOWN ? 2 * PH_DOWN : kTabMoeSlot + 1]);
  g.np = rfl(tab_wg[DOWN ? 2 * PH_DOWN + 1 : kTabMoeSlot + 2]) - g.p0;
  const int K = (DOWN ? P.Fe : P.d) / (MX ? 2 : 1);     // a row's bytes inside one expert
  g.npc = (K + 1023) >> 10;                             // 1 KB pieces per expert row
  g.tail = (K - 1024 * (g.npc - 1)) >> 4;               // lanes with codes in the last piece
  g.nsl = DOWN ? P.topk : 1;                            // experts per row pair
  g.per = g.nsl * g.npc;
  int u1;
  streamer_range(g.np * g.per, g.per, kStreamers, s, g.u0, u1);
  g.n = u1 - g.u0;
  return g;
}

// Issue cursor over a streamer's units: row pair t (from p0), expert segment
// sl, piece c; units past the share read zeros (out-of-range offsets), so the
// loads in flight never change in number.
struct MoeCur {
  int t, sl, c, issued;
};
__device__ __forceinline__ MoeCur moe_cursor(const MoeGeo& g, int u) {
  MoeCur c;
  c.t = u / g.per;
  c.sl = (u - c.t * g.per) / g.npc;
  c.c = u - c.t * g.per - c.sl * g.npc;
  c.issued = 0;
  return c;
}
// MXFP4: a lane's 16 bytes of a row are one 32-weight block, whose E8M0
// scale is one byte of the scale image (rs; 2 per unit, in s0 and s1).
template <bool DOWN, bool MX>
__device__ __forceinline__ void moe_issue(const Params& P, const MoeGeo& g, rsrc_t r, rsrc_t rs, const int* sel,
                                          int eslot, MoeCur& c, u32x4& b0, u32x4& b1, uint32_t& s0,
                                          uint32_t& s1) {
  const int lane = threadIdx.x & 63;
  const uint32_t row_bytes = (uint32_t)((DOWN ? P.Fe : P.d) / (MX ? 2 : 1));
  const int e = DOWN ? rfl(sel[c.sl]) : eslot;
  const uint32_t row = DOWN ? (uint32_t)(e * P.d + 2 * (g.p0 + c.t)) : (uint32_t)((e * P.Fe + g.p0 + c.t) * 2);
  const uint32_t row0 = (DOWN ? (uint32_t)P.e8_d : 0u) + row * row_bytes;
  const bool ok = c.issued < g.n && (c.c + 1 < g.npc || lane < g.tail);
  const uint32_t o = row0 + 1024u * (uint32_t)c.c + (uint32_t)lane * 16u;
  b0 = ld_nt(r, ok ? o : kOOB);
  b1 = ld_nt(r, ok ? o + row_bytes : kOOB + 16u);   // distinct: always two loads
  if (MX) {
    const uint32_t blocks = row_bytes / 16u;   // scales per row
    const uint32_t so = (DOWN ? (uint32_t)P.xsc_d : 0u) + row * blocks + 64u * (uint32_t)c.c + (uint32_t)lane;
    s0 = __builtin_amdgcn_raw_buffer_load_b8(rs, ok ? so : kOOB, 0, 0);
    s1 = __builtin_amdgcn_raw_buffer_load_b8(rs, ok ? so + blocks : kOOB + 16u, 0, 0);
  }
  ++c.issued;
  if (++c.c == g.npc) {
    c.c = 0;
    if (++c.sl == g.nsl) { c.sl = 0; ++c.t; }
  }
}

// Units a streamer keeps in flight in the routed phases.  Traced moe2b steps
// (E4M3 / MXFP4): 2 units 1.172 / 1.158 ms, 3 units 1.151 / 1.167 ms, 4 units
// 1.165 / 1.177 ms, 8 units 1.240 / 1.243 ms.
constexpr int kMoeUnits = 3;
// Streams the share with kMoeUnits units in flight in b.  Row sums go
// to out by ds_add, at most two contributors per row pair
// (streamer_range).  A down row's sum over one expert is scaled by that
// row's scale before the next expert's is added.  sel: this wave's routing
// words.  (Issuing the down phase's first units ahead, at the end of the GU
// stream or before the down phase's barrier, made the step slower: 1.35 and
// 1.22 against 1.16 ms traced on moe2b.)
template <bool DOWN, bool MX>
__device__ __forceinline__ void moe_stream(const Params& P, int l, int s, const int* tab_wg, const int* sel,
                                           int eslot, const float* sc_lds, const float* xs, float* out,
                                           u32x4 (&b)[2 * kMoeUnits]) {
  const int lane = threadIdx.x & 63;
  const MoeGeo g = moe_geo<DOWN, MX>(P, s, tab_wg);
  const rsrc_t r = make_rsrc(P.w8 + (size_t)rfl(l) * P.e8_stride, (uint32_t)P.e8_stride);
  const rsrc_t rs = make_rsrc(P.xsc + (size_t)rfl(l) * P.xsc_stride, MX ? (uint32_t)P.xsc_stride : 0u);
  uint32_t bs[2 * kMoeUnits];   // MXFP4: the units' block scales
  MoeCur ic = moe_cursor(g, g.u0);
#pragma unroll
  for (int k = 0; k < kMoeUnits; ++k)
    moe_issue<DOWN, MX>(P, g, r, rs, sel, eslot, ic, b[2 * k], b[2 * k + 1], bs[2 * k], bs[2 * k + 1]);
  int ct = ic.t, csl = 0, cc = 0;
  {
    const MoeCur c0 = moe_cursor(g, g.u0);
    ct = c0.t; csl = c0.sl; cc = c0.c;
  }
  float a0 = 0.f, a1 = 0.f, s0 = 0.f, s1 = 0.f;
  const int n = g.n;
  const int ngroups = (n + kMoeUnits - 1) / kMoeUnits;
  for (int grp = 0; grp < ngroups; ++grp) {
#pragma unroll
    for (int k = 0; k < kMoeUnits; ++k) {
      // (MXFP4: four loads per unit -- codes, then scales -- all in issue order)
      wait_vm<(MX ? 2 : 1) * (2 * kMoeUnits) - (MX ? 4 : 2)>();
      const int j = grp * kMoeUnits + k;
      if (j < n) {
        if (MX) {
          // a lane's 32 weights of the piece; lanes past the row's end skip
          if (cc + 1 < g.npc || lane < g.tail)
            dot32_mxfp4x2(b[2 * k], b[2 * k + 1], e8m0_float(bs[2 * k]), e8m0_float(bs[2 * k + 1]),
                          xs + (DOWN ? csl * P.Fe : 0) + 2048 * cc + 32 * lane, a0, a1);
        } else {
          dot16_e4m3x2(b[2 * k], b[2 * k + 1], xs + (DOWN ? csl * P.Fe : 0) + 1024 * cc + 16 * lane, a0, a1);
        }
        const bool last = j == n - 1, seg_end = cc + 1 == g.npc;
        if (DOWN && MX && (seg_end || last)) {
          s0 += a0;   // MXFP4: the block scales are applied already
          s1 += a1;
          a0 = a1 = 0.f;
        }
        if (DOWN && !MX && (seg_end || last)) {
          s0 = __builtin_fmaf(a0, sc_lds[csl * 2 * g.np + 2 * ct], s0);
          s1 = __builtin_fmaf(a1, sc_lds[csl * 2 * g.np + 2 * ct + 1], s1);
          a0 = a1 = 0.f;
        }
        if ((seg_end && csl + 1 == g.nsl) || last) {
          const float y0 = wave_sum(DOWN ? s0 : a0), y1 = wave_sum(DOWN ? s1 : a1);
          if (lane == 0) {
            lds_add(out + (DOWN ? 0 : kMoeOutPairs) + 2 * ct, y0);
            lds_add(out + (DOWN ? 0 : kMoeOutPairs) + 2 * ct + 1, y1);
          }
          a0 = a1 = s0 = s1 = 0.f;
        }
        if (++cc == g.npc) { cc = 0; if (++csl == g.nsl) { csl = 0; ++ct; } }
      }
      moe_issue<DOWN, MX>(P, g, r, rs, sel, eslot, ic, b[2 * k], b[2 * k + 1], bs[2 * k], bs[2 * k + 1]);
    }
  }
  wait_vm0();   // the zero-reading loads past the share's end
}

// Streamer role (waves 1..7): kBlocksInFlight loads always in flight, in
// stream order.  Every phase is a whole number of groups of kUnitsInFlight
// units (zero-reading units pad it), so unit k of each group always sits in
// register slot k: the steps below are unrolled over the slots and never
// copy a register that a load is still filling.
template <int HD, bool MOE>
__device__ __forceinline__ void streamer_role(const Params& P, const Launch& A, int g0, int g1, const int* tab,
                                              float* xs, float* out, const float* gs, float* red, const int* si,
                                              float* aux, float* sink, const int* tab_wg) {
  const int lane = threadIdx.x & 63;
  const uint32_t lane16 = (uint32_t)lane * 16u;
  Cursor cu;
  cursor_start(P, A, g0, g1, tab, cu);
  u32x4 mb[2 * kMoeUnits];   // mixture of experts: the routed phases' loads
  u32x4 buf[kBlocksInFlight];
#pragma unroll
  for (int k = 0; k < kUnitsInFlight; ++k) issue_unit(cu, lane16, buf[2 * k], buf[2 * k + 1]);
  PhaseIt id = phase_at(P, A, g0);
  for (; id.g < g1; phase_next(P, A, id)) {
    if (id.ph == -2) continue;
    if (id.ph == PH_ATTN) {
      if (!streamer_attention<1, HD>(P, A, id, si, aux, tab, sink)) break;
      continue;
    }
    __syncthreads();   // S1a
    if (si[12] == 0) break;
    float rv[kRouterChunk];   // mixture of experts, GU: the router-logit shares in flight
    if (MOE && id.ph == PH_GU) moe_router_issue(P, rv);
    if (norm_phase(id)) apply_gains(xs, gs, P.d, red);
    if (MOE && id.ph == PH_GU) moe_router_finish(P, rv, aux + kAuxRouter);
    __syncthreads();   // S1
    if (is_gemv(id.ph)) {
      const int* e = tab + id.ph * kTabStride;
      const int n = rfl(e[T_LEFT]);
      const int ngroups = (n + rfl(e[T_PAD])) / kUnitsInFlight;
      const int npc = rfl(e[T_NPC]);
      int t = rfl(e[T_T0]), col = rfl(e[T_COL]);
      float a0 = 0.f, a1 = 0.f;
      int u = 0;
      for (int grp = 0; grp < ngroups; ++grp) {
        // the issue side runs one group ahead; phases hold whole groups, so
        // it can only reach the end of its phase here
        if (cu.left == 0 && cu.pad == 0 && cu.it.g < g1) cursor_next(P, A, g1, tab, cu);
#pragma unroll
        for (int k = 0; k < kUnitsInFlight; ++k) {
          wait_vm<kBlocksInFlight - 2>();
          if (u < n) {
            const float* xl = xs + 8 * lane + 512 * col;
            const f32x4 xa = *reinterpret_cast<const f32x4*>(xl);
            const f32x4 xb = *reinterpret_cast<const f32x4*>(xl + 4);
            a0 = dot8(buf[2 * k], xa, xb, a0);
            a1 = dot8(buf[2 * k + 1], xa, xb, a1);
            if (col == npc - 1 || u == n - 1) {
              const float y0 = wave_sum(a0), y1 = wave_sum(a1);
              if (lane == 0) {   // at most two contributors (streamer_units)
                lds_add(out + 2 * t, y0);
                lds_add(out + 2 * t + 1, y1);
              }
              a0 = a1 = 0.f;
              ++t;
            }
            if (++col == npc) col = 0;
          }
          ++u;
          issue_unit(cu, lane16, buf[2 * k], buf[2 * k + 1]);
        }
      }
    }
    if constexpr (MOE) {
      if (id.ph == PH_GU) {
        // (S1 above: every wave's sum of the router-logit shares is in LDS)
        const int w = rfl((int)(threadIdx.x >> 6));
        float* rt = aux + kAuxRoute + 16 * w;
        moe_route(P, aux + kAuxRouter, red, rt);
        const int* sel = reinterpret_cast<const int*>(rt);
        const int eslot = rfl(sel[rfl(tab_wg[kTabMoeSlot])]);
        if (P.mx) moe_stream<false, true>(P, id.l, w, tab_wg, sel, eslot, nullptr, xs, out, mb);
        else moe_stream<false, false>(P, id.l, w, tab_wg, sel, eslot, nullptr, xs, out, mb);
      } else if (id.ph == PH_DOWN) {
        const int w = rfl((int)(threadIdx.x >> 6));
        const int* sel = reinterpret_cast<const int*>(aux) + kAuxRoute + 16 * w;
        if (P.mx) moe_stream<true, true>(P, id.l, w, tab_wg, sel, 0, aux + kAuxMoe, xs, out, mb);
        else moe_stream<true, false>(P, id.l, w, tab_wg, sel, 0, aux + kAuxMoe, xs, out, mb);
      }
    }
    __syncthreads();   // S2
  }
  wait_vm0();   // the zero-filled loads past the stream's end
}

// Streamer role of the batched kernel (waves 1..7): the same walk over the
// phases, but the stream is 1 KB weight tiles, kTilesInFlight in flight, and
// each tile is one MFMA.  Lane l supplies the B operand for sequence
// (l % 16) mod MB at k offset 8 (l / 16): 8 fp16 inputs from LDS.  Columns
// 8..15 repeat sequences 0..7 and columns of absent sequences hold stale
// inputs; neither is published.  A 16-row group's fp32 accumulator goes into
// LDS (ds_add_f32, per sequence) when the group or the streamer's range ends.
template <int MB, int HD>
__device__ __forceinline__ void streamer_tiles(const Params& P, const Launch& A, int g0, int g1, const int* tab,
                                               float* xs, float* out, float* slot, const float* gs, float* red,
                                               const int* si, float* aux, const int* plan, const float* slots) {
  static_assert(MB == 8, "the MFMA B operand maps columns to sequences mod 8");
  const int lane = threadIdx.x & 63, B = P.B;
  const uint32_t lane16 = (uint32_t)lane * 16u;
  const int col = lane & 15, kseg = lane >> 4, seq = col & (MB - 1);
  TileCursor cu;
  tcursor_start(P, A, g0, g1, tab, cu);
  u32x4 buf[kTilesInFlight];
#pragma unroll
  for (int k = 0; k < kTilesInFlight; ++k) issue_tile(cu, lane16, k, buf[k]);
  PhaseIt id = phase_at(P, A, g0);
  for (; id.g < g1; phase_next(P, A, id)) {
    if (id.ph == -2) continue;
    if (id.ph == PH_ATTN) {
      if (!streamer_attention<MB, HD>(P, A, id, si, aux)) break;
      continue;
    }
    __syncthreads();   // S1a
    if (si[12] == 0) break;
    if (dma_input(id)) {
      const int w = rfl((int)(threadIdx.x >> 6));
      dma_input_share<MB>(P, id, xs, w);
      if (norm_phase(id)) ss_share(P, w, red);
      wait_vm0();
    }
    __syncthreads();   // S1b: the phase input is in LDS
    // the embedded layer-0 input: x times the gains here (the others came
    // multiplied from their producers)
    if (norm_phase(id) && !dma_input(id))
      apply_gains_batch(reinterpret_cast<_Float16*>(xs), xs + kMaxBatch * gemv_span(P.d) / 2, gs, P.d, B, red);
    __syncthreads();   // S1
    if (is_gemv(id.ph)) {
      const int* e = tab + id.ph * kTabStride;
      const int n = rfl(e[T_LEFT]);
      const int ngroups = (n + rfl(e[T_PAD])) / kTilesInFlight;
      const int kt = rfl(e[T_NPC]);
      const int t0 = rfl(e[T_T0]), u0 = t0 * kt + rfl(e[T_COL]), u1 = u0 + n;
      int t = t0, j = rfl(e[T_COL]);
      // columns 32 j + 8 kseg .. + 7 of sequence seq (8-row blocks, blk8)
      const _Float16* xb = reinterpret_cast<const _Float16*>(xs) + blk8(seq, 8 * kseg);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      int u = 0;
      for (int grp = 0; grp < ngroups; ++grp) {
        if (cu.left == 0 && cu.pad == 0 && cu.it.g < g1) tcursor_next(P, A, g1, tab, cu);
#pragma unroll
        for (int k = 0; k < kTilesInFlight; ++k) {
          wait_vm<kTilesInFlight - 1>();
          if (u < n) {
            const f16x8 bv = *reinterpret_cast<const f16x8*>(xb + kTileCols * kMaxBatch * j);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, buf[k]), bv, acc, 0, 0, 0);
            if (++j == kt || u == n - 1) {
              if (col < B) {
                // rows 4 kseg .. 4 kseg + 3 of the group, sequence col
                float* o = (whole_group(t, kt, u0, u1) ? out + kTileRows * MB * t
                                                       : slot + (t == t0 ? 0 : kTileRows * MB)) +
                           4 * kseg * MB + col;
                const float c0 = acc[0], c1 = acc[1], c2 = acc[2], c3 = acc[3];
                o[0] = c0;
                o[MB] = c1;
                o[2 * MB] = c2;
                o[3 * MB] = c3;
              }
              acc = f32x4{0.f, 0.f, 0.f, 0.f};
              if (j == kt) { j = 0; ++t; }
            }
          }
          ++u;
          issue_tile(cu, lane16, k, buf[k]);
        }
      }
    }
    __syncthreads();   // S2
    if (is_gemv(id.ph)) {
      combine_all<MB>(id.ph, plan, slots, out);
      __syncthreads();   // S2b
    }
  }
  wait_vm0();   // the zero-filled loads past the stream's end
}

template <int MB, int HD, bool MOE = false>
__device__ __forceinline__ void dec_body(const Params& P, const Launch& A) {
  using M = Lds<MB>;
  extern __shared__ __attribute__((aligned(16))) float smem[];
  float* xs = smem;                                   // input region (see Lds)
  float* out = smem + M::Out;
  float* xown = smem + M::Own;
  float* red = smem + M::Red;
  float* scl = smem + M::Scl;
  int* si = reinterpret_cast<int*>(smem + M::Si);
  float* aux = smem + M::Aux;
  float* gs = smem + M::Gain;
  int* tab_wg = reinterpret_cast<int*>(smem + M::TabWg);
  // wave index through readfirstlane: provably uniform, so the role split
  // below is a scalar branch and every per-wave value stays in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  int* tab_all = reinterpret_cast<int*>(smem + M::Tab);
  int* tab = tab_all + (wave > 0 ? (wave - 1) * kStreamerTab : 0);
  float* slots = smem + M::Slot;
  int* plan = reinterpret_cast<int*>(smem + M::Plan);
  const int total = A.n_tok * phases_per_token(P.L);
  const int g0 = A.phase_begin < 0 ? 0 : A.phase_begin;
  const int g1 = A.phase_end < total ? A.phase_end : total;
  const int B = P.B;
  // MB > 1: where the normed phases' fp32 inputs are staged (after the fp16 ones)
  float* stage = xs + kMaxBatch * gemv_span(P.d) / 2;

  if constexpr (MB == 1) fill_tables(P, wave, tab_wg, tab);
  else fill_tables_tiled(P, wave, tab_wg, tab);
  wait_lgkm0();
  __syncthreads();   // every streamer's tables are in LDS
  if (wave > 0) {
    if constexpr (MB == 1)
      streamer_role<HD, MOE>(P, A, g0, g1, tab, xs, out, gs, red, si, aux, smem + M::Sink, tab_wg);
    else streamer_tiles<MB, HD>(P, A, g0, g1, tab, xs, out, slots + (wave - 1) * 2 * M::SlotN, gs, red, si, aux,
                                plan, slots);
    return;
  }
  if constexpr (MB > 1) {
    build_plans(tab_all, plan);
    wait_lgkm0();
  }

  // wave 0: control
  uint64_t* trace = P.trace ? P.trace + (size_t)blockIdx.x * P.trace_stride : nullptr;
  int ev = 0;
  auto stamp = [&]() {
    if (DEC_COLD(trace != nullptr) && lane == 0 && ev < P.trace_stride) st_g(trace + ev, wall_clock64());
    ++ev;
  };
  const int own = kOwnFloats / MB;   // xown floats per sequence
  {
    // this workgroup's rows of each sequence's residual stream
    int r0, r1;
    own_rows<MB>(P, r0, r1);
    for (int b = 0; b < B; ++b)
      for (int r = r0 + lane; r < r1; r += 64) xown[b * own + r - r0] = ld_coh(P.x + (size_t)b * P.d + r);
  }
  uint32_t epoch = A.bar_base;
  bool first = true, have_tok = false, gains_ready = false;
  // server launch: the next request when read ahead, whether the current
  // token's logits go to the host, and workgroup 0's unpublished completion
  Request rq;
  rq.state = 0;
  bool cur_lg = false;
  int done_pending = 0;
  int tok_local[MB];
#pragma unroll
  for (int b = 0; b < MB; ++b) tok_local[b] = 0;
  int prev_ph = -3, prev_i = 0, prev_l = 0;
  if (lane < kMaxBatch) scl[lane] = 1.0f;
  PhaseIt id = phase_at(P, A, g0);
  for (; id.g < g1; phase_next(P, A, id)) {
    if (id.ph == -2) continue;
    const int pos = step_pos(P, A, id.i);
    // outputs of the previous phase; this phase's LDS results start at zero
    if (!first) {
      if constexpr (MB > 1)
        if (is_gemv(prev_ph)) {
          combine_all<MB>(prev_ph, plan, slots, out);
          __syncthreads();   // S2b
        }
      // (the batched kernel stores the residual only where a launch ends)
      w0_store_outputs<MB, MOE>(P, prev_ph, prev_l, step_pos(P, A, prev_i), A.pos_end, tab_wg,
                                lg_mode(A, prev_i, cur_lg), scl, out, xown, aux, gs,
                                reinterpret_cast<const uint16_t*>(smem + M::MoeWr), MB == 1);
    }
    if (MB == 1 && is_gemv(id.ph)) {
      // the batch-1 streamers add into out (ds_add); the batched kernel's
      // streamers and combine store every live element
      const int np = rfl(tab_wg[2 * id.ph + 1]) - rfl(tab_wg[2 * id.ph]);
      for (int t = lane; t < 2 * np * MB; t += 64) out[t] = 0.f;
      if (MOE && id.ph == PH_GU) {
        // and the expert's gate/up row pairs after the router's logits
        const int nq = rfl(tab_wg[kTabMoeSlot + 2]) - rfl(tab_wg[kTabMoeSlot + 1]);
        for (int t = lane; t < 2 * nq; t += 64) out[kMoeOutPairs + t] = 0.f;
      }
    }
    const bool skip_bar = first || (id.ph == PH_QKV && id.l == 0 && have_tok);
    if (!skip_bar) {
      ++epoch;
      if (DEC_COLD(P.stress)) stress_delay(epoch);
      w0_arrive(P, A.fenced);
      // server launch: the previous request's tokens have landed with this
      // arrival's wait; its completion can go out
      if (DEC_COLD(A.server) && blockIdx.x == 0) srv_flush_done(P, done_pending);
      if constexpr (MB == 1 && !MOE)
        if (id.ph == PH_O && P.H > (int)gridDim.x / 32 && (int)blockIdx.x / wg_per_head(P, pos) >= P.H)
          w0_warm_gu(P, tab_all, id.l, smem + M::Sink);
      if constexpr (MB > 1)
        if (id.ph == PH_O && !P.cols_pos && (int)blockIdx.x / wg_per_head(P, pos) >= P.B * P.H)
          w0_warm_tiles(P, tab_all, id.l, smem + M::Sink);
    }
    auto wait = [&]() { return skip_bar ? true : w0_wait(P, epoch, A.fenced); };
    // the norm gains do not depend on the barrier: they were prefetched
    // during the previous normed phase, else start them now
    if (norm_phase(id)) {
      if (!gains_ready) w0_dma_vec(gs, norm_gains(P, id), P.d, 4, false);
      gains_ready = false;
    }
    if constexpr (MB > 1) {
      // the O and down outputs are published multiplied by the next norm's
      // gains; a launch that did not run the normed phase before fetches them
      if ((id.ph == PH_O || id.ph == PH_DOWN) && !gains_ready) {
        const float* gn = id.ph == PH_O ? P.gains + ((size_t)id.l * 2 + 1) * P.d
                                        : P.gains + (size_t)min(2 * (id.l + 1), 2 * P.L) * P.d;
        w0_dma_vec(gs, gn, P.d, 4, false);
        gains_ready = true;
      }
    }
    bool ok = true;
    if (id.ph == PH_ATTN) {
      // the streamers take attention units too: release them (S1a) right
      // after the grid barrier, then run this wave's own units
      auto wait_attn = [&]() {
        const bool r = wait();
        if (lane == 0) si[12] = r ? 1 : 0;
        __syncthreads();   // S1a
        return r;
      };
      ok = attention_wg<HD, MB>(P, id.l, pos, A.pos_end, 0, wg_per_head(P, pos), wait_attn, aux + kAuxPart);
      wait_vm0();   // this wave's stores are complete before the next arrive
      first = false;
      if (DEC_COLD(!ok)) return;
    } else if (id.ph == PH_QKV && id.l == 0) {
      ok = wait();
      bool forced = A.n_force && id.i == 0;
      if (DEC_COLD(A.server) && ok) {
        // a server launch: token i is request i, or the launch ends here
        if (rq.state == 0) {
          if (blockIdx.x == 0) srv_flush_done(P, done_pending);   // the host may be waiting for it
          srv_request(P, A, (uint32_t)id.i, true, rq);
        }
        ok = rq.state > 0;
        forced = (rq.flags & kReqForce) != 0;
        cur_lg = (rq.flags & kReqLogits) != 0;
        rq.state = 0;
        if (!ok && blockIdx.x == 0) srv_flush_done(P, done_pending);
      }
      if (ok) {
#pragma unroll
        for (int b = 0; b < MB; ++b) {
          if (b < B) {
            int tok;
            if (A.tok_src == TOK_PROMPT) {
              if (!P.cols_pos) tok = ldg(P.prompt + (size_t)b * A.n_tok + id.i);
              else tok = pos + b < A.pos_end ? ldg(P.prompt + (pos + b - A.pos0)) : 0;
            }
            else if (forced) tok = A.server ? rq.tok[b] : A.force[b];   // teacher forcing
            else tok = have_tok ? tok_local[b] : ld_coh(P.tok_cur + b);
            tok = tok < 0 ? 0 : (tok >= P.V ? P.V - 1 : tok);
            w0_embed<MB>(P, b, tok, MB == 1 ? xs : stage + (size_t)b * gemv_span(P.d), xown, own);
          }
        }
      }
      have_tok = false;
    } else if (id.ph == PH_QKV || id.ph == PH_GU || id.ph == PH_LM) {
      ok = wait();
      // (mixture of experts: zeros up to the next 1 KB piece of E4M3 codes)
      if constexpr (MB == 1)
        if (ok) w0_dma_vec(xs, P.x, P.d, 4, true, MOE ? 512 : 0);
    } else if (id.ph == PH_DOWN) {
      ok = wait();
      if constexpr (MB == 1)
        if (ok) w0_dma_vec(xs, P.act, P.F, 4, true, MOE ? 1024 : 0);

    } else if (id.ph == PH_O) {
      ok = wait();
      // the attention output of every head, merged in the attention phase
      if constexpr (MB == 1)
        if (ok) w0_dma_vec(xs, P.att_o, P.q, 4, true);
    } else {
      ok = wait();
      if (ok) {
        w0_argmax<MB>(P, id.i, P.cols_pos ? min(A.pos_end - 1 - pos, B - 1) : -1, tok_local);
        have_tok = true;
        if (DEC_COLD(A.server) && blockIdx.x == 0) srv_post_tokens<MB>(P, (uint32_t)id.i, tok_local, done_pending);
      }
    }
    if (id.ph != PH_ATTN) {
      wait_vm0();   // batch 1: the phase input has landed in LDS
      if (lane == 0) si[12] = ok ? 1 : 0;
      first = false;
      __syncthreads();   // S1a
      if (DEC_COLD(!ok)) return;
      if constexpr (MB > 1) {
        // batched: every wave lands its share of the inputs of all sequences
        if (dma_input(id)) {
          dma_input_share<MB>(P, id, xs, 0);
          if (norm_phase(id)) ss_share(P, 0, red);
          wait_vm0();
        }
        __syncthreads();   // S1b
      }
    }
    float rv[kRouterChunk];   // mixture of experts, GU: the router-logit shares in flight
    if (MOE && id.ph == PH_GU) moe_router_issue(P, rv);
    if (norm_phase(id)) {
      if constexpr (MB == 1) apply_gains(xs, gs, P.d, red);
      else if (!dma_input(id)) apply_gains_batch(reinterpret_cast<_Float16*>(xs), stage, gs, P.d, B, red);
    }
    if (MOE && id.ph == PH_GU) moe_router_finish(P, rv, aux + kAuxRouter);
    __syncthreads();   // S1
    if (DEC_COLD(P.stress)) w0_poison<MB>(P, id.ph, id.l, tab_wg);
    if (id.ph == PH_ATTN) w0_merge_wg<MB>(P, pos, A.pos_end, wg_per_head(P, pos), aux + kAuxPart);
    if (id.ph == PH_QKV) {
      // the rotary rows of this step's positions, for publishing q and k
      const int ncols = P.cols_pos ? min(B, P.max_ctx - pos) : 1;
      w0_dma_vec(aux, P.rope + (size_t)pos * P.hd, ncols * P.hd, 4, false);
      if constexpr (MOE) {
        // the router's columns of this workgroup's residual rows for the O
        // publication's router-logit shares, [E][rows] in fp16 pairs: dword
        // e * np + j holds rows r0 + 2j, r0 + 2j + 1 of expert e (landed with
        // the rotary rows, which the QKV publication waits for)
        const int r0 = 2 * rfl(tab_wg[2 * PH_O]), np = rfl(tab_wg[2 * PH_O + 1]) - rfl(tab_wg[2 * PH_O]);
        const rsrc_t r = make_rsrc(P.w + (size_t)id.l * P.layer_stride + P.off_gu, (uint32_t)(P.E * P.d * 2));
        for (int i0 = 0; i0 < P.E * np; i0 += 64) {
          const int i = i0 + lane, e = i / max(np, 1);
          const uint32_t off = i < P.E * np ? (uint32_t)(e * P.d + r0 + 2 * (i - e * np)) * 2u : kOOB;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(smem + M::MoeWr + i0), 4, off, 0, 0, 0);
        }
      }
    }
    if (norm_phase(id)) {
      // every wave has applied this phase's gains: fetch the next normed
      // phase's into the same LDS while this GEMV runs
      PhaseIt nx = id;
      do {
        phase_next(P, A, nx);
      } while (nx.g < g1 && !norm_phase(nx));
      if (nx.g < g1) {
        w0_dma_vec(gs, norm_gains(P, nx), P.d, 4, false);
        gains_ready = true;
      }
    }
    // this phase's norm scale per sequence, used when its outputs are published
    if (lane < kMaxBatch) {
      float s = 1.0f;
      if (norm_phase(id) && lane < B) {
        float ss = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) ss += red[lane * kWaves + w];
        s = 1.0f / sqrtf(ss / (float)P.d + P.eps);
      }
      scl[lane] = s;
    }
    if constexpr (MOE) {
      if (id.ph == PH_GU) {
        // (S1 above: every wave's sum of the router-logit shares is in LDS)
        // wave 0's routing words stay in LDS for the publication and the
        // down phase; workgroup 0 records the routing of the step's position
        moe_route(P, aux + kAuxRouter, red, aux + kAuxRoute);
        const int* route = reinterpret_cast<const int*>(aux) + kAuxRoute;
        if (blockIdx.x == 0 && lane < P.topk)
          st_coh(P.routes + ((size_t)pos * P.L + id.l) * P.topk + lane, route[lane]);
        // the row scales of this workgroup's down-phase output pairs in every
        // chosen expert, [slot][2 np], for the down phase's streamers (they
        // land while the experts' gate/up rows stream)
        const int r0 = 2 * rfl(tab_wg[2 * PH_DOWN]), nr = 2 * rfl(tab_wg[2 * PH_DOWN + 1]) - r0;
        const float* sd = P.esc + (size_t)id.l * P.sc_stride + P.sc_d;
        for (int i = lane; i < (P.mx ? 0 : P.topk * nr); i += 64) {
          const int k = i / nr;
          aux[kAuxMoe + i] = ldg(sd + (size_t)route[k] * P.d + r0 + (i - k * nr));
        }
      }
    }
    // server launch: read the next request ahead, while the streamers run --
    // workgroup 0 from the host early in the token, the others from their
    // device slot in the LM head, long after workgroup 0 has filled it
    if (DEC_COLD(A.server) && rq.state == 0 && id.i + 1 < A.n_tok &&
        ((blockIdx.x == 0 && ((id.ph == PH_GU && id.l == 0) || id.ph == PH_LM)) || (blockIdx.x != 0 && id.ph == PH_LM)))
      srv_request(P, A, (uint32_t)id.i + 1u, false, rq);
    stamp();
    __syncthreads();   // S2
    stamp();
    prev_ph = id.ph;
    prev_i = id.i;
    prev_l = id.l;
  }
  if (!first) {
    if constexpr (MB > 1)
      if (is_gemv(prev_ph)) {
        combine_all<MB>(prev_ph, plan, slots, out);
        __syncthreads();   // S2b
      }
    w0_store_outputs<MB, MOE>(P, prev_ph, prev_l, step_pos(P, A, prev_i), A.pos_end, tab_wg,
                              lg_mode(A, prev_i, cur_lg), scl, out, xown, aux, gs,
                              reinterpret_cast<const uint16_t*>(smem + M::MoeWr));
  }
  if (DEC_COLD(A.server) && blockIdx.x == 0) srv_flush_done(P, done_pending);
  wait_vm0();
}

// One kernel per head dimension (the attention code is specialised for it,
// and a kernel holding one variant is a fraction of the code the instruction
// cache has to serve): batch 1 and batched, for head_dim 8, 16, 32, 64, 128.
#define DEC_KERNELS(HD)                                                                                     \
  extern "C" __global__ __launch_bounds__(kThreads, 1) void dec_resident_hd##HD(const Params* __restrict__ Pp, \
                                                                                 Launch A) {                  \
    dec_body<1, HD>(*Pp, A);                                                                                \
  }                                                                                                         \
  extern "C" __global__ __launch_bounds__(kThreads, 1) void dec_resident_batch_hd##HD(                         \
      const Params* __restrict__ Pp, Launch A) {                                                            \
    dec_body<kMaxBatch, HD>(*Pp, A);                                                                        \
  }                                                                                                         \
  extern "C" __global__ __launch_bounds__(kThreads, 1) void dec_resident_moe_hd##HD(                           \
      const Params* __restrict__ Pp, Launch A) {                                                            \
    dec_body<1, HD, true>(*Pp, A);                                                                          \
  }
DEC_KERNELS(8)
DEC_KERNELS(16)
DEC_KERNELS(32)
DEC_KERNELS(64)
DEC_KERNELS(128)
#undef DEC_KERNELS

namespace {
// The kernel for a batch size and head dimension; nullptr for an unsupported head dimension.
const void* kernel_for(int kind, int hd) {
  const bool b = kind > 1;
  if (kind == kMoeKernel) {
    switch (hd) {
      case 8: return (const void*)dec_resident_moe_hd8;
      case 16: return (const void*)dec_resident_moe_hd16;
      case 32: return (const void*)dec_resident_moe_hd32;
      case 64: return (const void*)dec_resident_moe_hd64;
      case 128: return (const void*)dec_resident_moe_hd128;
      default: return nullptr;
    }
  }
  switch (hd) {
    case 8: return b ? (const void*)dec_resident_batch_hd8 : (const void*)dec_resident_hd8;
    case 16: return b ? (const void*)dec_resident_batch_hd16 : (const void*)dec_resident_hd16;
    case 32: return b ? (const void*)dec_resident_batch_hd32 : (const void*)dec_resident_hd32;
    case 64: return b ? (const void*)dec_resident_batch_hd64 : (const void*)dec_resident_hd64;
    case 128: return b ? (const void*)dec_resident_batch_hd128 : (const void*)dec_resident_hd128;
    default: return nullptr;
  }
}
}  // namespace

// Plain streaming read for the stream ceiling: the buffer's 1 KB blocks are
// split evenly over the grid's waves, and each wave reads its contiguous
// range with 16-byte non-temporal loads, eight blocks in flight (the access
// pattern of the decode kernel's weight streams).  Each thread stores the XOR
// of what it read so no load is dead.  n16 is a multiple of 64.
extern "C" __global__ __launch_bounds__(kThreads) void dec_stream_read(const u32x4* __restrict__ src, uint64_t n16,
                                                                       uint32_t* __restrict__ out) {
  const uint64_t nw = (uint64_t)gridDim.x * kWaves, nblk = n16 / 64;
  const uint64_t w = (uint64_t)blockIdx.x * kWaves + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  const uint64_t b1 = (w + 1) * nblk / nw;
  uint64_t b = w * nblk / nw;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; b + 8 <= b1; b += 8) {
    u32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = __builtin_nontemporal_load(src + (b + k) * 64 + lane);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= v[k];
  }
  for (; b < b1; ++b) acc ^= __builtin_nontemporal_load(src + b * 64 + lane);
  out[(uint64_t)blockIdx.x * kThreads + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

int kernel_stream_read(const void* src, uint64_t n16, uint32_t* out, int grid) {
  hipLaunchKernelGGL(dec_stream_read, dim3(grid), dim3(kThreads), 0, 0, static_cast<const u32x4*>(src), n16, out);
  return (int)hipGetLastError();
}

// Scratch of the no-allocation handle (dec_init_noalloc), for callers that
// cannot allocate device memory: one fixed array per device that holds a
// handle's exchange vectors, partial results, barrier counters and parameter
// blocks, kept until the process ends.  In host code the array's name is not
// a device address: the runtime is asked for that address once per device
// (with the device current), and only the pointer it returns is used --
// inside the parameter block the kernels receive, and for clearing.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

int kernel_scratch(int device, void** out) {
  static void* addr[kMaxDevices] = {};
  static std::mutex mu;
  if (device < 0 || device >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p) return (int)hipErrorInvalidSymbol;
    addr[device] = p;
  }
  *out = addr[device];
  return (int)hipSuccess;
}

int kernel_prepare() {
  for (int hd = 8; hd <= 128; hd *= 2)
    for (int kind : {1, kMaxBatch, kMoeKernel}) {
      const hipError_t e = hipFuncSetAttribute(kernel_for(kind, hd), hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
      if (e != hipSuccess) return (int)e;
    }
  return (int)hipSuccess;
}

int kernel_blocks_per_cu(int kind, int hd, int* out) {
  const void* k = kernel_for(kind, hd);
  if (!k) return (int)hipErrorInvalidValue;
  return (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(out, k, kThreads, kLdsBytes);
}

int kernel_launch_resident(const Params* P, const Launch& A, int grid, int kind, int hd, void* stream) {
  const void* k = kernel_for(kind, hd);
  if (!k) return (int)hipErrorInvalidValue;
  const Params* p = P;
  Launch a = A;
  void* args[] = {&p, &a};
  return (int)hipLaunchCooperativeKernel(k, dim3(grid), dim3(kThreads), args, kLdsBytes, static_cast<hipStream_t>(stream));
}

int kernel_launch_plain(const Params* P, const Launch& A, int grid, int kind, int hd, void* stream) {
  const void* k = kernel_for(kind, hd);
  if (!k) return (int)hipErrorInvalidValue;
  const Params* p = P;
  Launch a = A;
  void* args[] = {&p, &a};
  return (int)hipLaunchKernel(k, dim3(grid), dim3(kThreads), args, kLdsBytes, static_cast<hipStream_t>(stream));
}

}  // namespace decmono
