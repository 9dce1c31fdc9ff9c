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

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 ld_nt(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAuxNt);
}
__device__ __forceinline__ u32x4 ld_kv(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAuxNt | kAuxSc1);
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
// grid barrier
// ---------------------------------------------------------------------------
// epoch: cumulative barrier number (1-based, wrapping).  Returns false when the
// launch must stop (watchdog expired here or an error was raised elsewhere).
__device__ __noinline__ bool grid_barrier(const Params* __restrict__ Pp, uint32_t epoch, int fenced, int* s_flag) {
  const Params& P = *Pp;
  // This wave's coherent stores must have completed before the workgroup arrives.
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0) {
    if (fenced) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t G = gridDim.x;
    const uint32_t grp = blockIdx.x % kGroups;
    const uint32_t ngroups = G < (uint32_t)kGroups ? G : (uint32_t)kGroups;
    const uint32_t gsize = (G - grp + kGroups - 1) / kGroups;
    uint32_t* gcnt = P.ctl + kCtlGroup0 + 64 * grp;
    const uint32_t old = __hip_atomic_fetch_add(gcnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == gsize * epoch - 1u)
      __hip_atomic_fetch_add(P.ctl + kCtlGlobal, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t target = ngroups * epoch;
    int ok = 1;
    const uint64_t t0 = wall_clock64();
    while ((int)(ld_coh(P.ctl + kCtlGlobal) - target) < 0) {
      if (ld_coh(P.ctl + kCtlErr) != 0u) { ok = 0; break; }
      if (wall_clock64() - t0 > (uint64_t)P.watchdog_ticks) {
        uint32_t expected = 0u;
        __hip_atomic_compare_exchange_strong(P.ctl + kCtlErr, &expected, (uint32_t)kDevErrTimeout,
                                             __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = 0;
        break;
      }
    }
    if (fenced) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *s_flag = ok;
  }
  __syncthreads();
  return *s_flag != 0;
}

// ---------------------------------------------------------------------------
// GEMV: y = W x over row pairs [p0, p1) of a row-major fp16 matrix W[rows, K].
// Wave w takes pairs p0+w, p0+w+8, ...; lane l reads 16-byte pieces l, l+64, ...
// of both rows (NP pieces per lane cover K <= 512*NP).  xs: fp32 x in LDS,
// zero-padded to 512*NP.  epi(pair, y0, y1, lane) sees the reduced sums.
// ---------------------------------------------------------------------------
template <int NP, class Epi>
__device__ __forceinline__ void gemv_pairs(const uint16_t* W, int rows, int K, int p0, int p1,
                                           const float* xs, Epi& epi) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t row_bytes = (uint32_t)K * 2u;
  const rsrc_t r = make_rsrc(W, (uint32_t)rows * row_bytes);
  const int P16 = K >> 3;
  for (int pr = p0 + wave; pr < p1; pr += kWaves) {
    const uint32_t b0 = (uint32_t)(2 * pr) * row_bytes;
    u32x4 w0[NP], w1[NP];
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const int c = lane + 64 * k;
      const bool in = c < P16;
      w0[k] = ld_nt(r, in ? b0 + 16u * c : kOOB);
      w1[k] = ld_nt(r, in ? b0 + row_bytes + 16u * c : kOOB);
    }
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const f32x4* xp = reinterpret_cast<const f32x4*>(xs + 8 * (lane + 64 * k));
      const f32x4 xa = xp[0], xb = xp[1];
      a0 = dot8(w0[k], xa, xb, a0);
      a1 = dot8(w1[k], xa, xb, a1);
    }
    a0 = wave_sum(a0);
    a1 = wave_sum(a1);
    epi(pr, a0, a1, lane);
  }
}

// Pieces per lane of the instantiation gemv() uses for row length K.
__device__ __forceinline__ int gemv_np(int K) {
  const int np = (K + 511) >> 9;
  if (np <= 6) return np < 1 ? 1 : np;
  if (np <= 8) return 8;
  if (np <= 10) return 10;
  if (np <= 12) return 12;
  if (np <= 14) return 14;
  return 16;
}
// LDS floats of the input vector a GEMV with row length K reads (zero-padded past K).
__device__ __forceinline__ int gemv_span(int K) { return 512 * gemv_np(K); }

template <class Epi>
__device__ void gemv(const uint16_t* W, int rows, int K, int p0, int p1, const float* xs, Epi& epi) {
  const int np = gemv_np(K);
  if (np <= 1) gemv_pairs<1>(W, rows, K, p0, p1, xs, epi);
  else if (np <= 2) gemv_pairs<2>(W, rows, K, p0, p1, xs, epi);
  else if (np <= 3) gemv_pairs<3>(W, rows, K, p0, p1, xs, epi);
  else if (np <= 4) gemv_pairs<4>(W, rows, K, p0, p1, xs, epi);
  else if (np <= 5) gemv_pairs<5>(W, rows, K, p0, p1, xs, epi);
  else if (np <= 6) gemv_pairs<6>(W, rows, K, p0, p1, xs, epi);
  else if (np <= 8) gemv_pairs<8>(W, rows, K, p0, p1, xs, epi);
  else if (np <= 10) gemv_pairs<10>(W, rows, K, p0, p1, xs, epi);
  else if (np <= 12) gemv_pairs<12>(W, rows, K, p0, p1, xs, epi);
  else if (np <= 14) gemv_pairs<14>(W, rows, K, p0, p1, xs, epi);
  else gemv_pairs<16>(W, rows, K, p0, p1, xs, epi);
}

// ---------------------------------------------------------------------------
// prologues
// ---------------------------------------------------------------------------
// xs[0..gemv_span(n)) <- coherent copy of src[0..n), zero beyond n.  n % 4 == 0.
__device__ __forceinline__ void load_vec(float* xs, const float* src, int n) {
  const rsrc_t r = make_rsrc(src, (uint32_t)n * 4u);
  const int npad = gemv_span(n);
  for (int i = threadIdx.x * 4; i < npad; i += kThreads * 4)
    *reinterpret_cast<f32x4*>(xs + i) = ld_coh4(r, i < n ? (uint32_t)i * 4u : kOOB);
}

// RMSNorm in place: xs[i] = xs[i] / sqrt(mean(xs^2) + eps) * g[i] for i < n.
__device__ __forceinline__ void rmsnorm_lds(float* xs, int n, const float* g, float eps, float* red) {
  __syncthreads();
  float ss = 0.f;
  for (int i = threadIdx.x; i < n; i += kThreads) ss += xs[i] * xs[i];
  ss = block_sum(ss, red);
  const float s = 1.0f / sqrtf(ss / (float)n + eps);
  for (int i = threadIdx.x; i < n; i += kThreads) xs[i] = xs[i] * s * g[i];
  __syncthreads();
}

// ---------------------------------------------------------------------------
// phases
// ---------------------------------------------------------------------------
struct Lds {
  float* xs;    // GEMV input vector, kMaxK floats
  float* red;   // 64 floats
  int* si;      // 16 ints
  float* aux;   // attention / merge scratch
};

__device__ __noinline__ void phase_qkv(const Params* __restrict__ Pp, int l, int tok, bool first_layer, const Lds& S) {
  const Params& P = *Pp;
  const int d = P.d;
  if (first_layer) {
    // x = E[tok]: every workgroup converts the row; each owns rows of x to store.
    const uint16_t* e = P.w + P.off_E + (size_t)tok * d;
    const _Float16* eh = reinterpret_cast<const _Float16*>(e);
    for (int i = threadIdx.x; i < gemv_span(d); i += kThreads) S.xs[i] = i < d ? (float)eh[i] : 0.f;
    __syncthreads();
    int b, e_;
    split(d / 2, blockIdx.x, gridDim.x, b, e_);
    for (int r = 2 * b + threadIdx.x; r < 2 * e_; r += kThreads) st_coh(P.x + r, S.xs[r]);
  } else {
    load_vec(S.xs, P.x, d);
  }
  rmsnorm_lds(S.xs, d, P.gains + (size_t)l * 2 * d, P.eps, S.red);
  int b, e;
  split(3 * P.q / 2, blockIdx.x, gridDim.x, b, e);
  float* out = P.qkv;
  auto epi = [out](int pr, float y0, float y1, int lane) {
    if (lane == 0) { st_coh(out + 2 * pr, y0); st_coh(out + 2 * pr + 1, y1); }
  };
  gemv(P.w + (size_t)l * P.layer_stride + P.off_qkv, 3 * P.q, d, b, e, S.xs, epi);
}

// Single-query attention of every head over positions 0..pos, split into
// chunks of positions; each (head, chunk) unit writes an unnormalised partial
// (running max m, sum of exp l, sum of exp * V) that the O phase merges.
template <int HD>
__device__ __noinline__ void phase_attn(const Params* __restrict__ Pp, int l, int pos, const Lds& S) {
  const Params& P = *Pp;
  constexpr int LP = HD / 8;             // lanes per position (16 B of K or V each)
  constexpr int PPW = 64 / LP;           // positions per wave per pass
  constexpr int PPB = PPW * kWaves;      // positions per workgroup per pass
  constexpr int NPG = kThreads / LP;     // position groups in the V pass
  float* qs = S.aux;                     // [HD] rotated, scaled query
  float* kn = qs + HD;                   // [HD] new key (fp16-rounded)
  float* vn = kn + HD;                   // [HD] new value (fp16-rounded)
  float* stat = vn + HD;                 // [4]
  float* sc = stat + 4;                  // [kChunkMax] scores, then exp weights
  float* red = sc + kChunkMax;           // [NPG * HD]
  const int ctx = pos + 1, H = P.H, G = gridDim.x;
  const int C = attn_chunks(ctx, H, G);
  const int CH = (ctx + C - 1) / C;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float scale = 1.0f / sqrtf((float)HD);
  const size_t head_elems = (size_t)P.max_ctx * HD;
  for (int u = blockIdx.x; u < H * C; u += G) {
    const int h = u / C, c = u % C;
    const int j0 = c * CH;
    const int j1 = min(ctx, j0 + CH);
    const bool has_new = j0 < ctx && j1 == ctx;
    uint16_t* kc = P.kv + ((size_t)(l * 2 + 0) * H + h) * head_elems;
    uint16_t* vc = P.kv + ((size_t)(l * 2 + 1) * H + h) * head_elems;
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
        const uint32_t kb = (uint32_t)__builtin_bit_cast(uint16_t, kr0) | ((uint32_t)__builtin_bit_cast(uint16_t, kr1) << 16);
        const uint32_t vb = (uint32_t)__builtin_bit_cast(uint16_t, vr0) | ((uint32_t)__builtin_bit_cast(uint16_t, vr1) << 16);
        st_coh(reinterpret_cast<uint32_t*>(kc + (size_t)pos * HD + 2 * i), kb);
        st_coh(reinterpret_cast<uint32_t*>(vc + (size_t)pos * HD + 2 * i), vb);
      }
    }
    __syncthreads();
    const rsrc_t rk = make_rsrc(kc, (uint32_t)(head_elems * 2));
    const rsrc_t rv = make_rsrc(vc, (uint32_t)(head_elems * 2));
    // scores s_j = q . K_j (q already carries 1/sqrt(hd))
    {
      const int sub = lane % LP, pidx = lane / LP;
      const f32x4 qa = *reinterpret_cast<const f32x4*>(qs + 8 * sub);
      const f32x4 qb = *reinterpret_cast<const f32x4*>(qs + 8 * sub + 4);
#pragma unroll 4
      for (int jb = j0 + wave * PPW; jb < j1; jb += PPB) {
        const int j = jb + pidx;
        float s = 0.f;
        if (j < j1) {
          if (j == pos) {
            const f32x4 ka = *reinterpret_cast<const f32x4*>(kn + 8 * sub);
            const f32x4 kb = *reinterpret_cast<const f32x4*>(kn + 8 * sub + 4);
            s = ka[0] * qa[0] + ka[1] * qa[1] + ka[2] * qa[2] + ka[3] * qa[3] +
                kb[0] * qb[0] + kb[1] * qb[1] + kb[2] * qb[2] + kb[3] * qb[3];
          } else {
            s = dot8(ld_kv(rk, (uint32_t)(j * HD + 8 * sub) * 2u), qa, qb, 0.f);
          }
        }
        s = group_sum<LP>(s);
        if (sub == 0 && j < j1) sc[j - j0] = s;
      }
    }
    __syncthreads();
    const int n = j1 - j0;
    if (wave == 0) {
      float m = -INFINITY;
      for (int t = lane; t < n; t += 64) m = fmaxf(m, sc[t]);
      m = wave_max(m);
      float ls = 0.f;
      for (int t = lane; t < n; t += 64) {
        const float e = expf(sc[t] - m);
        sc[t] = e;
        ls += e;
      }
      ls = wave_sum(ls);
      if (lane == 0) { stat[0] = m; stat[1] = ls; }
    }
    __syncthreads();
    // acc = sum_j exp(s_j - m) V_j
    {
      const int dg = threadIdx.x % LP, pg = threadIdx.x / LP;
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int j = j0 + pg; j < j1; j += NPG) {
        const float wj = sc[j - j0];
        if (j == pos) {
#pragma unroll
          for (int t = 0; t < 8; ++t) acc[t] += wj * vn[8 * dg + t];
        } else {
          const f16x8 v = __builtin_bit_cast(f16x8, ld_kv(rv, (uint32_t)(j * HD + 8 * dg) * 2u));
#pragma unroll
          for (int t = 0; t < 8; ++t) acc[t] = __builtin_fmaf(wj, (float)v[t], acc[t]);
        }
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) red[pg * HD + 8 * dg + t] = acc[t];
    }
    __syncthreads();
    if (threadIdx.x < HD) {
      float s = 0.f;
      for (int p = 0; p < NPG; ++p) s += red[p * HD + threadIdx.x];
      st_coh(P.part + ((size_t)h * P.max_chunks + c) * HD + threadIdx.x, s);
    }
    if (threadIdx.x == 0) {
      st_coh(P.pml + ((size_t)h * P.max_chunks + c) * 2, stat[0]);
      st_coh(P.pml + ((size_t)h * P.max_chunks + c) * 2 + 1, stat[1]);
    }
    __syncthreads();
  }
}

// o = merged attention output of every head -> x += Wo o on this workgroup's rows.
__device__ __noinline__ void phase_o(const Params* __restrict__ Pp, int l, int pos, const Lds& S) {
  const Params& P = *Pp;
  const int ctx = pos + 1, H = P.H, hd = P.hd, q = P.q;
  const int C = attn_chunks(ctx, H, gridDim.x);
  float* sf = S.aux;   // [H * C] merge factor of each chunk
  for (int h = threadIdx.x; h < H; h += kThreads) {
    const float* pm = P.pml + (size_t)h * P.max_chunks * 2;
    float M = -INFINITY;
    for (int c = 0; c < C; ++c) M = fmaxf(M, ld_coh(pm + 2 * c));
    float sum = 0.f;
    for (int c = 0; c < C; ++c) {
      const float m = ld_coh(pm + 2 * c);
      sum += (m == -INFINITY ? 0.f : expf(m - M)) * ld_coh(pm + 2 * c + 1);
    }
    const float inv = 1.0f / sum;
    for (int c = 0; c < C; ++c) {
      const float m = ld_coh(pm + 2 * c);
      sf[h * C + c] = (m == -INFINITY ? 0.f : expf(m - M)) * inv;
    }
  }
  __syncthreads();
  const rsrc_t rp = make_rsrc(P.part, (uint32_t)((size_t)H * P.max_chunks * hd * 4));
  for (int i = threadIdx.x * 4; i < gemv_span(q); i += kThreads * 4) {
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    if (i < q) {
      const int h = i / hd, j = i % hd;
      for (int c = 0; c < C; ++c)
        o += sf[h * C + c] * ld_coh4(rp, (uint32_t)(((size_t)h * P.max_chunks + c) * hd + j) * 4u);
    }
    *reinterpret_cast<f32x4*>(S.xs + i) = o;
  }
  __syncthreads();
  int b, e;
  split(P.d / 2, blockIdx.x, gridDim.x, b, e);
  float* x = P.x;
  auto epi = [x](int pr, float y0, float y1, int lane) {
    if (lane == 0) {
      st_coh(x + 2 * pr, ld_coh(x + 2 * pr) + y0);
      st_coh(x + 2 * pr + 1, ld_coh(x + 2 * pr + 1) + y1);
    }
  };
  gemv(P.w + (size_t)l * P.layer_stride + P.off_o, P.d, q, b, e, S.xs, epi);
}

__device__ __noinline__ void phase_gu(const Params* __restrict__ Pp, int l, const Lds& S) {
  const Params& P = *Pp;
  const int d = P.d;
  load_vec(S.xs, P.x, d);
  rmsnorm_lds(S.xs, d, P.gains + (size_t)l * 2 * d + d, P.eps, S.red);
  int b, e;
  split(P.F, blockIdx.x, gridDim.x, b, e);
  float* act = P.act;
  auto epi = [act](int pr, float g, float u, int lane) {
    if (lane == 0) st_coh(act + pr, g / (1.0f + expf(-g)) * u);
  };
  gemv(P.w + (size_t)l * P.layer_stride + P.off_gu, 2 * P.F, d, b, e, S.xs, epi);
}

__device__ __noinline__ void phase_down(const Params* __restrict__ Pp, int l, const Lds& S) {
  const Params& P = *Pp;
  load_vec(S.xs, P.act, P.F);
  __syncthreads();
  int b, e;
  split(P.d / 2, blockIdx.x, gridDim.x, b, e);
  float* x = P.x;
  auto epi = [x](int pr, float y0, float y1, int lane) {
    if (lane == 0) {
      st_coh(x + 2 * pr, ld_coh(x + 2 * pr) + y0);
      st_coh(x + 2 * pr + 1, ld_coh(x + 2 * pr + 1) + y1);
    }
  };
  gemv(P.w + (size_t)l * P.layer_stride + P.off_d, P.d, P.F, b, e, S.xs, epi);
}

// logits = W_lm rmsnorm(x, g_final); per-workgroup (max, lowest index).
__device__ __noinline__ void phase_lm(const Params* __restrict__ Pp, int write_logits, const Lds& S) {
  const Params& P = *Pp;
  const int d = P.d;
  load_vec(S.xs, P.x, d);
  rmsnorm_lds(S.xs, d, P.gains + (size_t)P.L * 2 * d, P.eps, S.red);
  int b, e;
  split(P.Vlm / 2, blockIdx.x, gridDim.x, b, e);
  float best = -INFINITY;
  int bidx = 0x7fffffff;
  float* lg = write_logits ? P.logits : nullptr;
  auto epi = [&best, &bidx, lg](int pr, float y0, float y1, int lane) {
    if (y0 > best) { best = y0; bidx = 2 * pr; }
    if (y1 > best) { best = y1; bidx = 2 * pr + 1; }
    if (lg != nullptr && lane == 0) { lg[2 * pr] = y0; lg[2 * pr + 1] = y1; }
  };
  gemv(P.w + P.off_lm, P.Vlm, d, b, e, S.xs, epi);
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
  __syncthreads();
}

// Greedy token = argmax over the workgroups' partials (lowest index on ties).
// Every workgroup computes it (it is the next token's input); workgroup 0
// publishes it.
__device__ __noinline__ int phase_argmax(const Params* __restrict__ Pp, int i, const Lds& S) {
  const Params& P = *Pp;
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
__device__ __forceinline__ void attn_dispatch(const Params* __restrict__ P, int l, int pos, const Lds& S) {
  phase_attn<HD>(P, l, pos, S);
}

extern "C" __global__ __launch_bounds__(kThreads, 1) void dec_resident(const Params* __restrict__ Pp, Launch A) {
  const Params& P = *Pp;
  extern __shared__ __attribute__((aligned(16))) float smem[];
  Lds S;
  S.xs = smem;
  S.red = smem + kMaxK;
  S.si = reinterpret_cast<int*>(smem + kMaxK + 64);
  S.aux = smem + kMaxK + 64 + 16;
  const int L = P.L;
  const int ppt = phases_per_token(L);
  const long long total = (long long)A.n_tok * ppt;
  long long g0 = A.phase_begin < 0 ? 0 : A.phase_begin;
  long long g1 = (long long)A.phase_end < total ? (long long)A.phase_end : total;
  uint32_t epoch = A.bar_base;
  bool first = true, have_tok = false;
  int tok_local = 0;
  for (long long g = g0; g < g1; ++g) {
    const int i = (int)(g / ppt), k = (int)(g % ppt);
    const bool lm = !A.lm_last_only || i == A.n_tok - 1;
    if (k >= kPhasesPerLayer * L && !lm) continue;
    const int pos = A.pos0 + i;
    const bool skip_bar = first || (k == 0 && have_tok);
    if (!skip_bar) {
      ++epoch;
      if (!grid_barrier(Pp, epoch, A.fenced, S.si)) return;
    }
    first = false;
    if (k < kPhasesPerLayer * L) {
      const int l = k / kPhasesPerLayer, ph = k % kPhasesPerLayer;
      if (ph == PH_QKV) {
        int tok = 0;
        if (l == 0) {
          if (A.tok_src == TOK_PROMPT) tok = P.prompt[i];
          else tok = have_tok ? tok_local : ld_coh(P.tok_cur);
          have_tok = false;
          tok = tok < 0 ? 0 : (tok >= P.V ? P.V - 1 : tok);
        }
        phase_qkv(Pp, l, tok, l == 0, S);
      } else if (ph == PH_ATTN) {
        switch (P.hd) {
          case 8: attn_dispatch<8>(Pp, l, pos, S); break;
          case 16: attn_dispatch<16>(Pp, l, pos, S); break;
          case 32: attn_dispatch<32>(Pp, l, pos, S); break;
          case 64: attn_dispatch<64>(Pp, l, pos, S); break;
          default: attn_dispatch<128>(Pp, l, pos, S); break;
        }
      } else if (ph == PH_O) {
        phase_o(Pp, l, pos, S);
      } else if (ph == PH_GU) {
        phase_gu(Pp, l, S);
      } else {
        phase_down(Pp, l, S);
      }
    } else if (k == kPhasesPerLayer * L) {
      phase_lm(Pp, A.write_logits && i == A.n_tok - 1, S);
    } else {
      tok_local = phase_argmax(Pp, i, S);
      have_tok = true;
    }
  }
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
