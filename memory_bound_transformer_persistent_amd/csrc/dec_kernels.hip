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
// GPU推論の速度制限要因：メモリ帯域幅).  Every GEMV here streams its rows with
// 16-byte non-temporal buffer loads (one 1 KB contiguous segment per wave
// instruction), keeps the activation vector in LDS as fp32, accumulates in
// fp32 and reduces across the wave with DPP.  No MFMA: at one token per step
// there is no dense contraction to feed it.
//
// Cross-workgroup data (residual stream, q/k/v, attention partials, SwiGLU
// output, KV-cache appends, argmax partials) is written with agent-coherent
// (sc1) stores and read with agent-coherent loads, so a barrier needs no L2
// write-back or invalidate: it waits for this workgroup's stores to complete,
// then arrives on a per-group counter whose last arriver bumps the global
// counter.  Weights are read-only for the whole launch and use plain
// non-temporal loads.
#include <hip/hip_runtime.h>
#include <math.h>

#include "dec_internal.h"

namespace decmono {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kAuxNt = 0x2;    // non-temporal: streamed once
constexpr int kAuxSc1 = 0x10;  // coherent at device (agent) scope
constexpr uint32_t kOOB = 0xFFFFFF00u;  // buffer offset past any region: loads read 0

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void;

// LDS map (floats): xs [kMaxK] | red [64] | si [16 ints] | aux [kAuxFloats] | pf [kWaves][kPfFloats]
constexpr int kPfBlocks = 12;                // 1 KB blocks of weights prefetched per wave
constexpr int kPfFloats = kPfBlocks * 256;
constexpr int kAuxFloats = 3072;
constexpr int kLdsRed = kMaxK, kLdsSi = kMaxK + 64, kLdsAux = kMaxK + 80, kLdsPf = kMaxK + 80 + kAuxFloats;
static_assert((kLdsPf + kWaves * kPfFloats) * 4 <= kLdsBytes, "LDS map exceeds the allocation");
static_assert(kLdsPf % 4 == 0, "prefetch buffer must be 16-byte aligned");
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
// 16 bytes per lane from a buffer straight into LDS at lds_base + 16*lane (wave-uniform base).
__device__ __forceinline__ void dma16(rsrc_t r, float* lds_base, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, off, 0, 0, kAuxNt);
}
__device__ __forceinline__ void wait_vm0() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
__device__ __forceinline__ f32x4 ld_coh4(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAuxSc1));
}
__device__ __forceinline__ float ld_coh(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_coh(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_coh(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// Sum over the workgroup; every thread gets the same value.  red: kWaves floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) s += red[w];
  __syncthreads();
  return s;
}

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

__device__ __forceinline__ void split(int n, int g, int G, int& b, int& e) {
  b = (int)((long long)n * g / G);
  e = (int)((long long)n * (g + 1) / G);
}
__device__ __forceinline__ int round512(int n) { return (n + 511) & ~511; }

// ---------------------------------------------------------------------------
// weight prefetch into LDS
// ---------------------------------------------------------------------------
// A GEMV phase's work for one workgroup: row pairs [p0, p1) of W[rows, K].
// Wave w consumes pairs p0+w, p0+w+8, ... as a stream of 1 KB blocks, block
// b = (2*j + r)*NP + k for its j-th pair, row r of the pair, piece-column k.
struct GemvWork {
  const uint16_t* W;
  int rows, K, p0, p1;
};

// A row pair is streamed in nch column chunks of np pieces per lane (np <= 8,
// nch*np*512 >= K), so no more than 8 16-byte pieces per row sit in registers.
__device__ __forceinline__ void gemv_shape(int K, int& np, int& nch) {
  const int pieces = (K + 511) >> 9;          // 16-byte pieces per lane per row
  nch = (pieces + 7) >> 3;
  np = (pieces + nch - 1) / nch;
}
// LDS floats of the input vector a GEMV with row length K reads (zero-padded past K).
__device__ __forceinline__ int gemv_span(int K) {
  int np, nch;
  gemv_shape(K, np, nch);
  return 512 * np * nch;
}

// Waves [w_first, 8) copy the first kPfBlocks blocks of every wave's stream
// into pf + w*kPfFloats with LDS-direct buffer loads (pieces past K read 0).
// Block b of wave w's stream is unit u = b / (2*np) (pair u / nch, column
// chunk u % nch), row (b / np) & 1 of the pair, piece b % np.  Whoever reads
// the blocks first waits for the issuing waves (vmcnt) and a workgroup sync.
__device__ __forceinline__ void prefetch_issue(const GemvWork& g, float* pf, int w_first) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (wave < w_first || g.W == nullptr) return;
  const int nis = kWaves - w_first;
  int np, nch;
  gemv_shape(g.K, np, nch);
  const uint32_t row_bytes = (uint32_t)g.K * 2u;
  const rsrc_t r = make_rsrc(g.W, (uint32_t)g.rows * row_bytes);
  const int P16 = g.K >> 3;
  for (int f = wave - w_first; f < kWaves * kPfBlocks; f += nis) {
    const int tw = f / kPfBlocks, b = f % kPfBlocks;
    const int u = b / (2 * np), rr = (b / np) & 1, kk = b % np;
    const int pr = g.p0 + tw + kWaves * (u / nch);
    if (pr >= g.p1) continue;
    const int c = lane + 64 * ((u % nch) * np + kk);
    const uint32_t off = c < P16 ? (uint32_t)(2 * pr + rr) * row_bytes + 16u * c : kOOB;
    dma16(r, pf + tw * kPfFloats + b * 256, off);
  }
}

// ---------------------------------------------------------------------------
// grid barrier, split in two halves
// ---------------------------------------------------------------------------
// Arrive: waves [0, n_store) wait for their coherent stores to complete
// (vmcnt: waves that only have prefetch loads in flight skip it), the
// workgroup syncs, and thread 0 adds one to its group's counter (group =
// blockIdx % 8).  Wait (wave 0): lanes 0..7 poll the eight group counters
// until each holds group_size * epoch, so a workgroup is released one
// atomic hop after the last arrival.  epoch is the cumulative barrier number
// (1-based, wrapping).  The wait returns false if the watchdog expires here
// or any workgroup raised an error.
__device__ __forceinline__ void barrier_arrive(const Params& P, uint32_t epoch, int fenced, int n_store) {
  if ((int)(threadIdx.x >> 6) < n_store) wait_vm0();
  __syncthreads();
  if (threadIdx.x == 0) {
    if (fenced) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_fetch_add(P.ctl + kCtlGroup0 + 64 * (blockIdx.x % kGroups), 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  }
}

__device__ __forceinline__ bool barrier_wait(const Params& P, uint32_t epoch, int fenced) {
  const int lane = threadIdx.x & 63;
  const uint32_t G = gridDim.x;
  const int ng = G < (uint32_t)kGroups ? (int)G : kGroups;
  uint32_t target = 0;
  const uint32_t* cnt = P.ctl + kCtlGroup0 + 64 * (lane < ng ? lane : 0);
  if (lane < ng) target = ((G - (uint32_t)lane + kGroups - 1) / kGroups) * epoch;
  const uint64_t t0 = wall_clock64();
  bool ok = true;
  while (true) {
    const bool done = lane >= ng || (int)(ld_coh(cnt) - target) >= 0;
    if (__all(done)) break;
    if (ld_coh(P.ctl + kCtlErr) != 0u) { ok = false; break; }
    if (wall_clock64() - t0 > (uint64_t)P.watchdog_ticks) {
      if (lane == 0) {
        uint32_t expected = 0u;
        __hip_atomic_compare_exchange_strong(P.ctl + kCtlErr, &expected, (uint32_t)kDevErrTimeout,
                                             __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      ok = false;
      break;
    }
  }
  if (fenced) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return ok;
}

// ---------------------------------------------------------------------------
// GEMV: y = W x over the row pairs of a GemvWork.  A wave's work is a stream of
// units (pair, column chunk); lane l reads 16-byte pieces l, l+64, ... of both
// rows of the unit, and the first kPfBlocks 1 KB blocks of the stream come from
// the LDS prefetch when pf is set.  While one unit is multiplied the next
// unit's loads are in flight.  xs: fp32 x in LDS, zero-padded to
// gemv_span(K).  epi(pair, y0, y1, lane) sees the wave-reduced sums.
// ---------------------------------------------------------------------------
template <int NP>
__device__ __forceinline__ void gemv_fetch(rsrc_t r, uint32_t row_bytes, int P16, int pr, int u, int ch,
                                           const float* pfw, int lane, u32x4 (&w0)[NP], u32x4 (&w1)[NP]) {
  const uint32_t b0 = (uint32_t)(2 * pr) * row_bytes;
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const int c = lane + 64 * (ch * NP + k);
    const bool in = c < P16;
    const int blk0 = (2 * u) * NP + k, blk1 = (2 * u + 1) * NP + k;
    if (pfw != nullptr && blk0 < kPfBlocks)
      w0[k] = *reinterpret_cast<const u32x4*>(pfw + blk0 * 256 + lane * 4);
    else
      w0[k] = ld_nt(r, in ? b0 + 16u * c : kOOB);
    if (pfw != nullptr && blk1 < kPfBlocks)
      w1[k] = *reinterpret_cast<const u32x4*>(pfw + blk1 * 256 + lane * 4);
    else
      w1[k] = ld_nt(r, in ? b0 + row_bytes + 16u * c : kOOB);
  }
}

template <int NP>
__device__ __forceinline__ void gemv_accum(const u32x4 (&w0)[NP], const u32x4 (&w1)[NP], const float* xs, int lane,
                                           int ch, float& a0, float& a1) {
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const f32x4* xp = reinterpret_cast<const f32x4*>(xs + 8 * (lane + 64 * (ch * NP + k)));
    const f32x4 xa = xp[0], xb = xp[1];
    a0 = dot8(w0[k], xa, xb, a0);
    a1 = dot8(w1[k], xa, xb, a1);
  }
}

template <int NP, class Epi>
__device__ __forceinline__ void gemv_stream(const GemvWork& g, int nch, const float* xs, const float* pf, Epi& epi) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t row_bytes = (uint32_t)g.K * 2u;
  const rsrc_t r = make_rsrc(g.W, (uint32_t)g.rows * row_bytes);
  const int P16 = g.K >> 3;
  const float* pfw = pf ? pf + wave * kPfFloats : nullptr;
  const int npairs = g.p1 - g.p0 - wave > 0 ? (g.p1 - g.p0 - wave + kWaves - 1) / kWaves : 0;
  const int nunits = npairs * nch;
  if (nunits == 0) return;
  float a0 = 0.f, a1 = 0.f;
  u32x4 x0[NP], x1[NP], y0[NP], y1[NP];
  auto pair_of = [&](int u) { return g.p0 + wave + kWaves * (u / nch); };
  gemv_fetch<NP>(r, row_bytes, P16, pair_of(0), 0, 0, pfw, lane, x0, x1);
  auto finish = [&](int u) {
    if (u % nch == nch - 1) {
      const float s0 = wave_sum(a0), s1 = wave_sum(a1);
      epi(pair_of(u), s0, s1, lane);
      a0 = 0.f;
      a1 = 0.f;
    }
  };
  for (int u = 0; u < nunits; u += 2) {
    if (u + 1 < nunits) gemv_fetch<NP>(r, row_bytes, P16, pair_of(u + 1), u + 1, (u + 1) % nch, pfw, lane, y0, y1);
    gemv_accum<NP>(x0, x1, xs, lane, u % nch, a0, a1);
    finish(u);
    if (u + 1 >= nunits) break;
    if (u + 2 < nunits) gemv_fetch<NP>(r, row_bytes, P16, pair_of(u + 2), u + 2, (u + 2) % nch, pfw, lane, x0, x1);
    gemv_accum<NP>(y0, y1, xs, lane, (u + 1) % nch, a0, a1);
    finish(u + 1);
  }
}

template <class Epi>
__device__ __forceinline__ void gemv(const GemvWork& g, const float* xs, const float* pf, Epi& epi) {
  int np, nch;
  gemv_shape(g.K, np, nch);
  switch (np) {
    case 1: gemv_stream<1>(g, nch, xs, pf, epi); break;
    case 2: gemv_stream<2>(g, nch, xs, pf, epi); break;
    case 3: gemv_stream<3>(g, nch, xs, pf, epi); break;
    case 4: gemv_stream<4>(g, nch, xs, pf, epi); break;
    case 5: gemv_stream<5>(g, nch, xs, pf, epi); break;
    case 6: gemv_stream<6>(g, nch, xs, pf, epi); break;
    case 7: gemv_stream<7>(g, nch, xs, pf, epi); break;
    default: gemv_stream<8>(g, nch, xs, pf, epi); break;
  }
}

// The GEMV work of each phase for this workgroup (pairs split evenly).
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
  split(npairs, blockIdx.x, gridDim.x, g.p0, g.p1);
  return g;
}

// ---------------------------------------------------------------------------
// prologues: run by wave 0 alone while the other waves' prefetch lands
// ---------------------------------------------------------------------------
constexpr int kVecBatch = 16;   // 16-byte loads per lane in flight in a prologue

// xs[0..gemv_span(n)) <- src[0..n) (coherent loads), zero past n; with g set,
// the RMSNorm of src times g: src / sqrt(mean(src^2) + eps) * g.
__device__ __forceinline__ void w0_load_vec(float* xs, const float* src, int n, const float* g, float eps) {
  const int lane = threadIdx.x & 63;
  const rsrc_t r = make_rsrc(src, (uint32_t)n * 4u);
  const int span = gemv_span(n);
  float ss = 0.f;
  for (int i0 = 0; i0 < span; i0 += 256 * kVecBatch) {
    f32x4 v[kVecBatch], gv[kVecBatch];
#pragma unroll
    for (int t = 0; t < kVecBatch; ++t) {
      const int i = i0 + 256 * t + 4 * lane;
      v[t] = ld_coh4(r, i < n ? (uint32_t)i * 4u : kOOB);
      if (g != nullptr) gv[t] = (i < n) ? *reinterpret_cast<const f32x4*>(g + i) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int t = 0; t < kVecBatch; ++t) {
      const int i = i0 + 256 * t + 4 * lane;
      if (i < span) {
        ss += v[t][0] * v[t][0] + v[t][1] * v[t][1] + v[t][2] * v[t][2] + v[t][3] * v[t][3];
        *reinterpret_cast<f32x4*>(xs + i) = g != nullptr ? v[t] * gv[t] : v[t];
      }
    }
  }
  if (g != nullptr) {
    const float s = 1.0f / sqrtf(wave_sum(ss) / (float)n + eps);
    for (int i = 4 * lane; i < n; i += 256) *reinterpret_cast<f32x4*>(xs + i) *= s;
  }
}

// Layer-0 input: x = E[tok] (fp16 -> fp32); this workgroup stores its own rows
// of x, and xs gets rmsnorm(x) * g.
__device__ __forceinline__ void w0_embed(const Params& P, int tok, float* xs, const float* g) {
  const int lane = threadIdx.x & 63, d = P.d;
  const _Float16* e = reinterpret_cast<const _Float16*>(P.w + P.off_E + (size_t)tok * d);
  int b, en;
  split(d / 2, blockIdx.x, gridDim.x, b, en);
  const int span = gemv_span(d);
  float ss = 0.f;
  for (int i = 8 * lane; i < span; i += 512) {
    f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
    if (i < d) {
      const f16x8 h = *reinterpret_cast<const f16x8*>(e + i);
      lo = f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
      hi = f32x4{(float)h[4], (float)h[5], (float)h[6], (float)h[7]};
      for (int q = 0; q < 8; ++q)
        if (i + q >= 2 * b && i + q < 2 * en) st_coh(P.x + i + q, q < 4 ? lo[q] : hi[q - 4]);
      const f32x4 ga = *reinterpret_cast<const f32x4*>(g + i), gb = *reinterpret_cast<const f32x4*>(g + i + 4);
      ss += lo[0] * lo[0] + lo[1] * lo[1] + lo[2] * lo[2] + lo[3] * lo[3] +
            hi[0] * hi[0] + hi[1] * hi[1] + hi[2] * hi[2] + hi[3] * hi[3];
      lo *= ga;
      hi *= gb;
    }
    *reinterpret_cast<f32x4*>(xs + i) = lo;
    *reinterpret_cast<f32x4*>(xs + i + 4) = hi;
  }
  const float s = 1.0f / sqrtf(wave_sum(ss) / (float)d + P.eps);
  for (int i = 4 * lane; i < d; i += 256) *reinterpret_cast<f32x4*>(xs + i) *= s;
}

// ---------------------------------------------------------------------------
// phases
// ---------------------------------------------------------------------------
struct Lds {
  float* xs;    // GEMV input vector, kMaxK floats
  float* red;   // 64 floats
  int* si;      // 16 ints
  float* aux;   // attention / argmax scratch, kAuxFloats
  float* pf;    // weight prefetch, kWaves x kPfFloats
};

// Single-query attention of every head over positions 0..pos, split into
// chunks of positions.  AW waves compute; a thread holds K and V of NPASS
// positions in registers (their loads are issued before the query is read),
// so a unit costs one memory round trip per group of GRP positions, with an
// online softmax across groups.  With more than one chunk per head each unit
// stores an unnormalised partial (max m, sum of exp l, sum of exp * V) and
// the last unit of a head to finish (per-head counter) merges them; the head's
// output o goes to P.attn_o.
template <int HD, int AW>
__device__ __forceinline__ void phase_attn(const Params& P, int l, int pos, const Lds& S) {
  constexpr int LP = HD / 8;             // lanes per position (16 B of K or V each)
  constexpr int PPW = 64 / LP;           // positions per wave per pass
  constexpr int PPB = PPW * AW;          // positions per workgroup per pass
  constexpr int NPASS = 4;
  constexpr int GRP = PPB * NPASS;       // positions per register group
  float* qs = S.aux;                     // [HD] rotated, scaled query
  float* kn = qs + HD;                   // [HD] new key (fp16-rounded)
  float* vn = kn + HD;                   // [HD] new value (fp16-rounded)
  float* wred = vn + HD;                 // [2 * kWaves]
  float* ored = wred + 2 * kWaves;       // [AW * HD]
  const int ctx = pos + 1, H = P.H, G = gridDim.x;
  const int C = attn_chunks(ctx, H, G);
  const int CH = (ctx + C - 1) / C;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool cw = wave < AW;
  const int sub = lane % LP, pidx = lane / LP;
  const float scale = 1.0f / sqrtf((float)HD);
  const size_t head_elems = (size_t)P.max_ctx * HD;
  for (int u = blockIdx.x; u < H * C; u += G) {
    const int h = u / C, c = u % C;
    const int j0 = c * CH;
    const int j1 = min(ctx, j0 + CH);
    const bool has_new = j0 < ctx && j1 == ctx;
    uint16_t* kc = P.kv + ((size_t)(l * 2 + 0) * H + h) * head_elems;
    uint16_t* vc = P.kv + ((size_t)(l * 2 + 1) * H + h) * head_elems;
    const rsrc_t rk = make_rsrc(kc, (uint32_t)(head_elems * 2));
    const rsrc_t rv = make_rsrc(vc, (uint32_t)(head_elems * 2));
    float M = -INFINITY, Lsum = 0.f;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int g0 = j0; g0 < j1; g0 += GRP) {
      u32x4 kr[NPASS], vr[NPASS];
      if (cw) {
#pragma unroll
        for (int t = 0; t < NPASS; ++t) {
          const int j = g0 + t * PPB + wave * PPW + pidx;
          const uint32_t off = (j < j1 && j != pos) ? (uint32_t)(j * HD + 8 * sub) * 2u : kOOB;
          kr[t] = ld_kv(rk, off);
          vr[t] = ld_kv(rv, off);
        }
      }
      if (g0 == j0) {
        if (threadIdx.x < HD / 2) {
          const int i = threadIdx.x;
          const float cs = P.rope[((size_t)pos * (HD / 2) + i) * 2];
          const float sn = P.rope[((size_t)pos * (HD / 2) + i) * 2 + 1];
          const float* qh = P.qkv + h * HD;
          const float q0 = ld_coh(qh + 2 * i), q1 = ld_coh(qh + 2 * i + 1);
          qs[2 * i] = (q0 * cs - q1 * sn) * scale;
          qs[2 * i + 1] = (q0 * sn + q1 * cs) * scale;
          if (has_new) {
            const float* kh = P.qkv + P.q + h * HD;
            const float* vh = P.qkv + 2 * P.q + h * HD;
            const float k0 = ld_coh(kh + 2 * i), k1 = ld_coh(kh + 2 * i + 1);
            const _Float16 kr0 = (_Float16)(k0 * cs - k1 * sn), kr1 = (_Float16)(k0 * sn + k1 * cs);
            const _Float16 vr0 = (_Float16)ld_coh(vh + 2 * i), vr1 = (_Float16)ld_coh(vh + 2 * i + 1);
            kn[2 * i] = (float)kr0; kn[2 * i + 1] = (float)kr1;
            vn[2 * i] = (float)vr0; vn[2 * i + 1] = (float)vr1;
            const uint32_t kb = (uint32_t)__builtin_bit_cast(uint16_t, kr0) |
                                ((uint32_t)__builtin_bit_cast(uint16_t, kr1) << 16);
            const uint32_t vb = (uint32_t)__builtin_bit_cast(uint16_t, vr0) |
                                ((uint32_t)__builtin_bit_cast(uint16_t, vr1) << 16);
            st_coh(reinterpret_cast<uint32_t*>(kc + (size_t)pos * HD + 2 * i), kb);
            st_coh(reinterpret_cast<uint32_t*>(vc + (size_t)pos * HD + 2 * i), vb);
          }
        }
        __syncthreads();
      }
      float s[NPASS];
      if (cw) {
        const f32x4 qa = *reinterpret_cast<const f32x4*>(qs + 8 * sub);
        const f32x4 qb = *reinterpret_cast<const f32x4*>(qs + 8 * sub + 4);
        float mloc = -INFINITY;
#pragma unroll
        for (int t = 0; t < NPASS; ++t) {
          const int j = g0 + t * PPB + wave * PPW + pidx;
          float dsum;
          if (j == pos) {
            const f32x4 ka = *reinterpret_cast<const f32x4*>(kn + 8 * sub);
            const f32x4 kb = *reinterpret_cast<const f32x4*>(kn + 8 * sub + 4);
            dsum = ka[0] * qa[0] + ka[1] * qa[1] + ka[2] * qa[2] + ka[3] * qa[3] +
                   kb[0] * qb[0] + kb[1] * qb[1] + kb[2] * qb[2] + kb[3] * qb[3];
          } else {
            dsum = dot8(kr[t], qa, qb, 0.f);
          }
          dsum = group_sum<LP>(dsum);
          s[t] = j < j1 ? dsum : -INFINITY;
          mloc = fmaxf(mloc, s[t]);
        }
        mloc = wave_max(mloc);
        if (lane == 0) wred[wave] = mloc;
      }
      __syncthreads();
      float mg = wred[0];
#pragma unroll
      for (int w = 1; w < AW; ++w) mg = fmaxf(mg, wred[w]);
      const float Mn = fmaxf(M, mg);
      const float alpha = M == -INFINITY ? 0.f : expf(M - Mn);
      if (cw) {
        float lloc = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[t] *= alpha;
#pragma unroll
        for (int t = 0; t < NPASS; ++t) {
          const int j = g0 + t * PPB + wave * PPW + pidx;
          const float e = j < j1 ? expf(s[t] - Mn) : 0.f;
          lloc += e;
          if (j == pos) {
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(e, vn[8 * sub + q], acc[q]);
          } else {
            const f16x8 v = __builtin_bit_cast(f16x8, vr[t]);
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(e, (float)v[q], acc[q]);
          }
        }
        // every lane of a position group holds the same e: count it once
        lloc = wave_sum(sub == 0 ? lloc : 0.f);
        if (lane == 0) wred[kWaves + wave] = lloc;
      }
      __syncthreads();
      float lg = 0.f;
#pragma unroll
      for (int w = 0; w < AW; ++w) lg += wred[kWaves + w];
      Lsum = Lsum * alpha + lg;
      M = Mn;
      __syncthreads();
    }
    // sum acc over the position groups of each wave, then over waves
    if (cw) {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        for (int off = LP; off < 64; off <<= 1) acc[q] += __shfl_xor(acc[q], off, 64);
      if (pidx == 0) {
#pragma unroll
        for (int q = 0; q < 8; ++q) ored[wave * HD + 8 * sub + q] = acc[q];
      }
    }
    __syncthreads();
    float o = 0.f;
    if (threadIdx.x < HD) {
#pragma unroll
      for (int w = 0; w < AW; ++w) o += ored[w * HD + threadIdx.x];
    }
    if (C == 1) {
      if (threadIdx.x < HD) st_coh(P.attn_o + h * HD + threadIdx.x, o / Lsum);
    } else {
      float* pp = P.part + ((size_t)h * P.max_chunks) * HD;
      float* pm = P.pml + ((size_t)h * P.max_chunks) * 2;
      if (threadIdx.x < HD) st_coh(pp + (size_t)c * HD + threadIdx.x, o);
      if (threadIdx.x == 0) { st_coh(pm + 2 * c, M); st_coh(pm + 2 * c + 1, Lsum); }
      if (cw) wait_vm0();
      __syncthreads();
      if (threadIdx.x == 0) {
        uint32_t* hc = P.ctl + kCtlHead0 + h;
        const uint32_t old = __hip_atomic_fetch_add(hc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = old == (uint32_t)(C - 1);
        if (last) st_coh(hc, 0u);   // every unit of this head has arrived: re-arm for the next layer
        S.si[10] = last;
      }
      __syncthreads();
      if (S.si[10] != 0 && threadIdx.x < HD) {
        // merge the C partials of head h with a running max
        constexpr int MB = 8;
        float Mr = -INFINITY, Lr = 0.f, Or = 0.f;
        for (int c0 = 0; c0 < C; c0 += MB) {
          float mv[MB], lv[MB], pv[MB];
#pragma unroll
          for (int t = 0; t < MB; ++t) {
            const bool in = c0 + t < C;
            mv[t] = in ? ld_coh(pm + 2 * (c0 + t)) : -INFINITY;
            lv[t] = in ? ld_coh(pm + 2 * (c0 + t) + 1) : 0.f;
            pv[t] = in ? ld_coh(pp + (size_t)(c0 + t) * HD + threadIdx.x) : 0.f;
          }
#pragma unroll
          for (int t = 0; t < MB; ++t) {
            if (mv[t] == -INFINITY) continue;
            const float Mn = fmaxf(Mr, mv[t]);
            const float a = Mr == -INFINITY ? 0.f : expf(Mr - Mn);
            const float bscale = expf(mv[t] - Mn);
            Or = Or * a + pv[t] * bscale;
            Lr = Lr * a + lv[t] * bscale;
            Mr = Mn;
          }
        }
        st_coh(P.attn_o + h * HD + threadIdx.x, Or / Lr);
      }
    }
    __syncthreads();
  }
}

// logits -> per-workgroup (max, lowest index) after phase LM's GEMV.
__device__ __forceinline__ void lm_finish(const Params& P, float best, int bidx, const Lds& S) {
  float* bv = S.red;
  int* bi = S.si;
  if ((threadIdx.x & 63) == 0) { bv[threadIdx.x >> 6] = best; bi[threadIdx.x >> 6] = bidx; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float v = bv[0];
    int ix = bi[0];
    for (int w = 1; w < kWaves; ++w)
      if (bv[w] > v || (bv[w] == v && bi[w] < ix)) { v = bv[w]; ix = bi[w]; }
    st_coh(P.amax_v + blockIdx.x, v);
    st_coh(P.amax_i + blockIdx.x, ix);
  }
}

// Greedy token = argmax over the workgroups' partials (lowest index on ties).
// Every workgroup computes it (it is the next token's input); workgroup 0
// publishes it.
__device__ __forceinline__ int phase_argmax(const Params& P, int i, const Lds& S) {
  float* v = S.aux;
  int* ix = reinterpret_cast<int*>(S.aux + 1024);
  const int G = gridDim.x;
  for (int t = threadIdx.x; t < G; t += kThreads) { v[t] = ld_coh(P.amax_v + t); ix[t] = ld_coh(P.amax_i + t); }
  __syncthreads();
  if (threadIdx.x < 64) {
    float bvv = -INFINITY;
    int bii = 0x7fffffff;
    for (int t = threadIdx.x; t < G; t += 64)
      if (v[t] > bvv || (v[t] == bvv && ix[t] < bii)) { bvv = v[t]; bii = ix[t]; }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bvv, off, 64);
      const int oi = __shfl_xor(bii, off, 64);
      if (ov > bvv || (ov == bvv && oi < bii)) { bvv = ov; bii = oi; }
    }
    if (threadIdx.x == 0) {
      const int tok = (bii == 0x7fffffff) ? 0 : bii;
      S.si[8] = tok;
      if (blockIdx.x == 0) { st_coh(P.tok_cur, tok); st_coh(P.tok_out + i, tok); }
    }
  }
  __syncthreads();
  return S.si[8];
}

template <int HD>
__device__ __forceinline__ void attn_dispatch(const Params& P, int l, int pos, int aw, const Lds& S) {
  if (aw == 4) phase_attn<HD, 4>(P, l, pos, S);
  else phase_attn<HD, kWaves>(P, l, pos, S);
}

// Attention positions per chunk up to which four waves compute it (and the
// other four prefetch the O projection meanwhile).
constexpr int kAttnNarrow = 64;

extern "C" __global__ __launch_bounds__(kThreads, 1) void dec_resident(const Params* __restrict__ Pp, Launch A) {
  const Params& P = *Pp;
  extern __shared__ __attribute__((aligned(16))) float smem[];
  Lds S;
  S.xs = smem;
  S.red = smem + kLdsRed;
  S.si = reinterpret_cast<int*>(smem + kLdsSi);
  S.aux = smem + kLdsAux;
  S.pf = smem + kLdsPf;
  const int wave = threadIdx.x >> 6;
  const int L = P.L, d = P.d;
  const int ppt = phases_per_token(L);
  const int nlayer_ph = kPhasesPerLayer * L;
  const long long total = (long long)A.n_tok * ppt;
  const long long g0 = A.phase_begin < 0 ? 0 : A.phase_begin;
  const long long g1 = (long long)A.phase_end < total ? (long long)A.phase_end : total;
  uint32_t epoch = A.bar_base;
  bool first = true, have_tok = false;
  int tok_local = 0;
  int n_store = kWaves;    // waves with coherent stores pending from the previous phase
  long long pf_for = -1;   // global index of the phase whose first weight blocks sit in S.pf
  uint64_t* trace = P.trace ? P.trace + (size_t)blockIdx.x * P.trace_stride : nullptr;
  int ev = 0;
  auto stamp = [&]() {
    if (trace && threadIdx.x == 0 && ev < P.trace_stride) trace[ev] = wall_clock64();
    ++ev;
  };
  for (long long g = g0; g < g1; ++g) {
    const int i = (int)(g / ppt), k = (int)(g % ppt);
    const bool lm = !A.lm_last_only || i == A.n_tok - 1;
    if (k >= nlayer_ph && !lm) continue;
    const int pos = A.pos0 + i;
    const int l = k < nlayer_ph ? k / kPhasesPerLayer : 0;
    const int ph = k < nlayer_ph ? k % kPhasesPerLayer : (k == nlayer_ph ? (int)PH_LM : -1);
    const bool is_gemv = ph == PH_QKV || ph == PH_O || ph == PH_GU || ph == PH_DOWN || ph == PH_LM;
    const bool skip_bar = first || (k == 0 && have_tok);
    bool ok = true;
    if (!skip_bar) {
      ++epoch;
      barrier_arrive(P, epoch, A.fenced, n_store);
      if (is_gemv && pf_for != g) {
        prefetch_issue(work_of(P, ph, l), S.pf, 1);
        pf_for = g;
      }
      if (wave == 0) ok = barrier_wait(P, epoch, A.fenced);
    }
    first = false;
    // prologue: wave 0 brings this phase's input vector into LDS
    int tok = 0;
    if (ph == PH_QKV && l == 0) {
      if (A.tok_src == TOK_PROMPT) tok = P.prompt[i];
      else tok = have_tok ? tok_local : ld_coh(P.tok_cur);
      have_tok = false;
      tok = tok < 0 ? 0 : (tok >= P.V ? P.V - 1 : tok);
    }
    if (wave == 0) {
      if (ph == PH_QKV) {
        if (l == 0) w0_embed(P, tok, S.xs, P.gains);
        else w0_load_vec(S.xs, P.x, d, P.gains + (size_t)l * 2 * d, P.eps);
      } else if (ph == PH_O) {
        w0_load_vec(S.xs, P.attn_o, P.q, nullptr, 0.f);
      } else if (ph == PH_GU) {
        w0_load_vec(S.xs, P.x, d, P.gains + (size_t)l * 2 * d + d, P.eps);
      } else if (ph == PH_DOWN) {
        w0_load_vec(S.xs, P.act, P.F, nullptr, 0.f);
      } else if (ph == PH_LM) {
        w0_load_vec(S.xs, P.x, d, P.gains + (size_t)L * 2 * d, P.eps);
      }
      if (threadIdx.x == 0) S.si[12] = ok ? 1 : 0;
    } else if (is_gemv) {
      wait_vm0();   // this wave's prefetch blocks have landed
    }
    __syncthreads();
    if (S.si[12] == 0) {
      wait_vm0();
      return;
    }
    stamp();
    const bool use_pf = pf_for == g;
    const float* pf = use_pf ? S.pf : nullptr;
    n_store = kWaves;
    if (ph == PH_QKV) {
      float* out = P.qkv;
      auto epi = [out](int pr, float y0, float y1, int lane) {
        if (lane == 0) { st_coh(out + 2 * pr, y0); st_coh(out + 2 * pr + 1, y1); }
      };
      gemv(work_of(P, PH_QKV, l), S.xs, pf, epi);
    } else if (ph == PH_ATTN) {
      const int ctx = pos + 1;
      const int C = attn_chunks(ctx, P.H, gridDim.x);
      const int aw = (ctx + C - 1) / C <= kAttnNarrow ? 4 : kWaves;
      if (aw == 4) {
        // the other four waves prefetch the O projection meanwhile
        prefetch_issue(work_of(P, PH_O, l), S.pf, 4);
        pf_for = g + 1;
        n_store = 4;
      }
      switch (P.hd) {
        case 8: attn_dispatch<8>(P, l, pos, aw, S); break;
        case 16: attn_dispatch<16>(P, l, pos, aw, S); break;
        case 32: attn_dispatch<32>(P, l, pos, aw, S); break;
        case 64: attn_dispatch<64>(P, l, pos, aw, S); break;
        default: attn_dispatch<128>(P, l, pos, aw, S); break;
      }
    } else if (ph == PH_O || ph == PH_DOWN) {
      float* x = P.x;
      auto epi = [x](int pr, float y0, float y1, int lane) {
        if (lane == 0) {
          st_coh(x + 2 * pr, ld_coh(x + 2 * pr) + y0);
          st_coh(x + 2 * pr + 1, ld_coh(x + 2 * pr + 1) + y1);
        }
      };
      gemv(work_of(P, ph, l), S.xs, pf, epi);
    } else if (ph == PH_GU) {
      float* act = P.act;
      auto epi = [act](int pr, float gt, float up, int lane) {
        if (lane == 0) st_coh(act + pr, gt / (1.0f + expf(-gt)) * up);
      };
      gemv(work_of(P, PH_GU, l), S.xs, pf, epi);
    } else if (ph == PH_LM) {
      float best = -INFINITY;
      int bidx = 0x7fffffff;
      float* lgp = (A.write_logits && i == A.n_tok - 1) ? P.logits : nullptr;
      auto epi = [&best, &bidx, lgp](int pr, float y0, float y1, int lane) {
        if (y0 > best) { best = y0; bidx = 2 * pr; }
        if (y1 > best) { best = y1; bidx = 2 * pr + 1; }
        if (lgp != nullptr && lane == 0) { lgp[2 * pr] = y0; lgp[2 * pr + 1] = y1; }
      };
      gemv(work_of(P, PH_LM, 0), S.xs, pf, epi);
      lm_finish(P, best, bidx, S);
    } else {
      tok_local = phase_argmax(P, i, S);
      have_tok = true;
    }
    stamp();
  }
  wait_vm0();   // no LDS-direct load may outlive the workgroup
}

int kernel_prepare() {
  return (int)hipFuncSetAttribute((const void*)dec_resident, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
}

int kernel_blocks_per_cu(int* out) {
  return (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(out, (const void*)dec_resident, kThreads, kLdsBytes);
}

int kernel_launch_resident(const Params* P, const Launch& A, int grid, void* stream) {
  const Params* p = P;
  Launch a = A;
  void* args[] = {&p, &a};
  return (int)hipLaunchCooperativeKernel((const void*)dec_resident, dim3(grid), dim3(kThreads), args, kLdsBytes,
                                         static_cast<hipStream_t>(stream));
}

int kernel_launch_plain(const Params* P, const Launch& A, int grid, void* stream) {
  hipLaunchKernelGGL(dec_resident, dim3(grid), dim3(kThreads), kLdsBytes, static_cast<hipStream_t>(stream), P, A);
  return (int)hipGetLastError();
}

}  // namespace decmono
