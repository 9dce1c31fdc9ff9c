// Matrix-form prefill for gfx950: every prompt position goes through each
// weight matrix in one pass, as matrix products on the matrix cores, instead
// of one position (or eight) per step of the decode kernel.
//
// The prompt phase sets the time to first token, one of the three speed
// figures the pages list for inference benchmarks beside throughput and
// per-request decode speed (hakusoku.com/story/7519, section
// 単一リクエストLLMデコード速度の重要性).  Over a whole prompt the products
// are dense: n positions times every weight, above the matrix cores' ridge
// (about 310 flop per HBM byte) once n passes a few hundred, so for long
// prompts the matrix cores and not HBM bound this path.
//
// Per layer, for the prompt positions pos0 .. pos0+n-1 with x their fp32
// residual rows:
//   h = fp16(x * g_attn), s = 1/rms(x)                        mp_norm
//   qkv = s * (h Wqkv^T); in its epilogue rotary on q and k,
//     k, v (fp16) to the KV cache, q (fp16) to q16               mp_gemm (ROPE)
//   o = causal softmax(q k^T) v over cache positions, fp16      mp_attention
//   x += o Wo^T                                                 mp_gemm (accumulate)
//   h = fp16(x * g_ffn), s = 1/rms(x)                         mp_norm
//   a = fp16(silu(gate) * up), gate, up = s * (h Wgu^T)        mp_gemm (SWIGLU)
//   x += a Wd^T                                                 mp_gemm (accumulate)
// then the final norm of the prompt's last position, its LM-head row and
// the argmax.  Matrix-product inputs are rounded to fp16 as in the batched
// decode kernel; q and the softmax weights are also rounded to fp16 for the
// attention products.  Every sum has a fixed order (split-K partials too), so
// results do not depend on timing.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "dec_internal.h"

namespace decmono {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4m __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc;
typedef __attribute__((address_space(3))) void lds_ptr;

constexpr uint32_t kOutOfRange = 0x80000000u;   // a buffer offset past every record: reads 0

__device__ __forceinline__ rsrc make_res(const void* base, uint64_t bytes) {
  const uint32_t n = bytes >= 0x7fffffffull ? 0x7fffffffu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)n, 0x00020000);
}
__device__ __forceinline__ f16x8 ld8(rsrc r, uint32_t off) {
  return __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// s_waitcnt vmcnt(N): at most N of this wave's vector-memory loads (LDS DMA
// included) still pending; they complete in issue order
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
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
// Wait until at most `later` K tiles' DMAs (PER loads each) are pending.
template <int PER, int NS>
__device__ __forceinline__ void wait_tiles(int later) {
  static_assert(PER * (NS - 2) < 64, "vmcnt is 6 bits");
  switch (later) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<PER * (NS >= 3)>(); break;
    case 2: wait_vmcnt<PER * 2 * (NS >= 4)>(); break;
    case 3: wait_vmcnt<PER * 3 * (NS >= 5)>(); break;
    case 4: wait_vmcnt<PER * 4 * (NS >= 6)>(); break;
    case 5: wait_vmcnt<PER * 5 * (NS >= 7)>(); break;
    default: wait_vmcnt<PER * 6 * (NS >= 8)>(); break;
  }
}
__device__ __forceinline__ float wave_sum64(float v) {
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// x[m][:] = E[tok[m]] in fp32 (tokens were range-checked by the host).  One
// workgroup per position.
__global__ __launch_bounds__(256) void mp_embed(const uint16_t* __restrict__ E, const int* __restrict__ tok, int d,
                                                float* __restrict__ x) {
  const int m = blockIdx.x;
  const _Float16* e = reinterpret_cast<const _Float16*>(E) + (size_t)tok[m] * d;
  for (int i = threadIdx.x; i < d; i += 256) x[(size_t)m * d + i] = (float)e[i];
}

// h[m] = fp16(x[m] * g) and s[m] = 1 / sqrt(mean(x[m]^2) + eps).  One
// workgroup per row, four consecutive elements per thread and access (d is a
// multiple of 32); the sum of squares is added per thread in index order,
// then over the wave, then over the four waves in order.
__global__ __launch_bounds__(256) void mp_norm(const float* __restrict__ x, const float* __restrict__ g, int d,
                                               float eps, uint16_t* __restrict__ h, float* __restrict__ s) {
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
  __shared__ float part[4];
  const int m = blockIdx.x, tid = threadIdx.x;
  const f32x4v* xr = reinterpret_cast<const f32x4v*>(x + (size_t)m * d);
  const f32x4v* gr = reinterpret_cast<const f32x4v*>(g);
  f16x4* hr = reinterpret_cast<f16x4*>(reinterpret_cast<_Float16*>(h) + (size_t)m * d);
  float ss = 0.f;
  for (int i = tid; i < d / 4; i += 256) {
    const f32x4v v = xr[i], gg = gr[i];
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    f16x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = (_Float16)(v[k] * gg[k]);
    hr[i] = o;
  }
  ss = wave_sum64(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  if (tid == 0) s[m] = 1.0f / sqrtf((part[0] + part[1] + part[2] + part[3]) / (float)d + eps);
}

// Epilogue of one result pair (columns n, n+1; n even) for the pair modes:
// v0, v1 are the scaled results.
__device__ __forceinline__ void pair_store(const MpEpi& e, int m, int n, float v0, float v1) {
  if (e.mode == MP_EP_SWIGLU) {
    reinterpret_cast<_Float16*>(e.H)[(size_t)m * e.ldh + (n >> 1)] = (_Float16)(v0 / (1.0f + expf(-v0)) * v1);
    return;
  }
  // rotary embedding and cache append: pairs (2i, 2i+1) of a head turn by the
  // angle in the cos/sin table row of the position
  const int part = n / e.q, rr = n - part * e.q, h = rr / e.hd, d = rr - h * e.hd, pos = e.pos0 + m;
  const size_t at = (size_t)h * e.head_elems + (size_t)pos * e.hd + d;
  if (part == 2) {
    reinterpret_cast<_Float16*>(e.vc)[at] = (_Float16)v0;
    reinterpret_cast<_Float16*>(e.vc)[at + 1] = (_Float16)v1;
    return;
  }
  const float* rt = e.rope + (size_t)pos * e.hd + d;
  const float cs = rt[0], sn = rt[1];
  const float z0 = __builtin_fmaf(v0, cs, -(v1 * sn)), z1 = __builtin_fmaf(v0, sn, v1 * cs);
  if (part == 0) {
    const float qscale = 1.0f / sqrtf((float)e.hd);
    _Float16* o = reinterpret_cast<_Float16*>(e.H) + (size_t)m * e.ldh + rr;
    o[0] = (_Float16)(z0 * qscale);
    o[1] = (_Float16)(z1 * qscale);
  } else {
    reinterpret_cast<_Float16*>(e.kc)[at] = (_Float16)z0;
    reinterpret_cast<_Float16*>(e.kc)[at + 1] = (_Float16)z1;
  }
}

// The epilogue of one wave's WM x WN result blocks: element (i, j, r) is row
// mrow + 16 i + 4 (lane / 16) + r and column ncol + 16 j + lane % 16.  Pair
// modes take the partner column from the neighbouring lane (every lane
// shuffles, then the even lanes store).
template <int WM, int WN>
__device__ __forceinline__ void wave_epilogue(const MpEpi& e, const f32x4m (&acc)[WM][WN], int mrow, int ncol, int M,
                                              int N, int lane) {
  const bool pair = e.mode == MP_EP_SWIGLU || e.mode == MP_EP_ROPE;
  float* Cz = e.mode == MP_EP_PART ? e.C + (size_t)blockIdx.z * M * N : e.C;
  const int ldc = e.mode == MP_EP_PART ? N : e.ldc;
#pragma unroll
  for (int i = 0; i < WM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = mrow + 16 * i + (lane >> 4) * 4 + r;
      const bool mok = m < M;
      const float sc = (e.mode != MP_EP_ACCUM && e.mode != MP_EP_PART && e.s && mok) ? e.s[m] : 1.0f;
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const int n = ncol + 16 * j + (lane & 15);
        const float v = acc[i][j][r] * sc;
        if (pair) {
          const float w = __shfl_xor(v, 1, 64);
          if (mok && n < N && !(n & 1)) pair_store(e, m, n, v, w);
          continue;
        }
        if (!mok || n >= N) continue;
        float* c = Cz + (size_t)m * ldc + n;
        if (e.mode == MP_EP_ACCUM) *c = *c + v;
        else *c = v;
      }
    }
  }
}

// C[M x N] from A [M x K] and B [N x K], both fp16 with K contiguous (row
// strides lda, ldb; K a multiple of 32): C = A B^T through the epilogue
// (MpEpilogue).  Four waves per workgroup in a WR x (4/WR) arrangement, each
// computing a (16 WM) x (16 WN) block as WM x WN products of
// v_mfma_f32_16x16x32_f16.  Operand layout of that instruction: lane l holds
// row l % 16 and the 8 K-elements 8 (l / 16) .. +7 of a 32-wide K step (a
// row of A for the A operand, a row of B -- a column of C -- for the B
// operand); the result is lane l's rows 4 (l / 16) .. +3 at column l % 16.
// Each lane loads its operands straight from the K-contiguous rows, 16 bytes
// per load, one K step ahead of the products; rows past M or N read as zero.
// Split z (blockIdx.z) covers K elements [z kc, min(K, (z+1) kc)).
template <int WM, int WN, int WR>
__global__ __launch_bounds__(256) void mp_gemm(const uint16_t* __restrict__ A, int lda, const uint16_t* __restrict__ B,
                                               int ldb, int M, int N, int K, int kc, MpEpi e) {
  constexpr int WC = 4 / WR;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = wave / WC, wc = wave % WC;
  const int m0 = blockIdx.y * (16 * WM * WR) + wr * 16 * WM, n0 = blockIdx.x * (16 * WN * WC) + wc * 16 * WN;
  const int kb = blockIdx.z * kc, ke = min(K, kb + kc);
  const rsrc ra = make_res(A, (uint64_t)M * lda * 2), rb = make_res(B, (uint64_t)N * ldb * 2);
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  uint32_t offa[WM], offb[WN];
#pragma unroll
  for (int i = 0; i < WM; ++i) {
    const int m = m0 + 16 * i + r16;
    offa[i] = m < M ? (uint32_t)((size_t)m * lda + kb + kq) * 2u : kOutOfRange;
  }
#pragma unroll
  for (int j = 0; j < WN; ++j) {
    const int n = n0 + 16 * j + r16;
    offb[j] = n < N ? (uint32_t)((size_t)n * ldb + kb + kq) * 2u : kOutOfRange;
  }
  f32x4m acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = f32x4m{0.f, 0.f, 0.f, 0.f};
  f16x8 a[WM], b[WN];
#pragma unroll
  for (int i = 0; i < WM; ++i) a[i] = ld8(ra, offa[i]);
#pragma unroll
  for (int j = 0; j < WN; ++j) b[j] = ld8(rb, offb[j]);
  for (int k = kb; k < ke; k += 32) {
    f16x8 an[WM], bn[WN];
    const bool more = k + 32 < ke;
    const uint32_t step = (uint32_t)(k + 32 - kb) * 2u;
#pragma unroll
    for (int i = 0; i < WM; ++i) an[i] = ld8(ra, more && offa[i] != kOutOfRange ? offa[i] + step : kOutOfRange);
#pragma unroll
    for (int j = 0; j < WN; ++j) bn[j] = ld8(rb, more && offb[j] != kOutOfRange ? offb[j] + step : kOutOfRange);
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < WM; ++i) a[i] = an[i];
#pragma unroll
    for (int j = 0; j < WN; ++j) b[j] = bn[j];
  }
  wave_epilogue<WM, WN>(e, acc, m0, n0, M, N, lane);
}

// One wave's share of K tile t of an LDS-staged product: PER 1 KB operand
// blocks (block wave + 4 j) into stage t % NS, one 16-byte LDS DMA per lane.
// roff is the lane's row offset at the split's first K element (kOutOfRange
// for rows past the matrix), kst the block's K step within the tile.
template <int PER, int NS, int STAGE>
__device__ __forceinline__ void dma_tile(char* lds, int t, int wave, int lane, rsrc ra, rsrc rb, const uint32_t* roff,
                                         const int* kst, const bool* isa, int kb, int ke) {
  char* st = lds + (t % NS) * STAGE;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int k0 = t * 64 + kst[j] * 32;   // from kb
    const uint32_t off = (roff[j] != kOutOfRange && kb + k0 < ke) ? roff[j] + (uint32_t)k0 * 2u : kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(isa[j] ? ra : rb, (lds_ptr*)(st + (wave + 4 * j) * 1024), 16, off, 0, 0,
                                             0);
  }
}

// The same product with both operands staged in LDS, for 17 to 128 rows
// (the weight-streaming products): BM x BN tiles, K in 64-wide tiles, NS
// tiles in flight.  A tile's
// operands land in LDS as 1 KB blocks already in the MFMA operand layout:
// block (r, s) holds rows 16 r .. +15 and K step s (32 wide) of the tile,
// lane l's 16 bytes at 16 l being row l % 16, K elements 8 (l / 16) .. +7.
// Each block is one 16-byte-per-lane LDS DMA of one wave
// (buffer_load ... lds), so the operand reads are linear ds_read_b128 with no
// bank conflicts and no register staging.  The four waves split the tile
// 2 x 2, each computing (BM/2) x (BN/2) with v_mfma_f32_16x16x32_f16.  Rows
// past M or N and K steps past the split's end load nothing useful (offsets
// past the buffer); their products are skipped or land in rows and columns
// that are not stored.
template <int BM, int BN, int NS>
__global__ __launch_bounds__(256) void mp_gemm_lds(const uint16_t* __restrict__ A, int lda,
                                                   const uint16_t* __restrict__ B, int ldb, int M, int N, int K, int kc,
                                                   MpEpi e) {
  constexpr int WM = BM / 32, WN = BN / 32;          // 16 x 16 blocks per wave
  constexpr int ABLK = BM / 16 * 2, BBLK = BN / 16 * 2;
  constexpr int NBLK = ABLK + BBLK, PER = NBLK / 4;  // DMA blocks per tile, per wave
  constexpr int STAGE = NBLK * 1024;
  static_assert(NBLK % 4 == 0, "blocks split evenly over the waves");
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  // the wave index in a scalar register: buffer descriptors and LDS bases chosen by it stay scalar
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  const int mb = blockIdx.y * BM, nb = blockIdx.x * BN;
  const int kb = blockIdx.z * kc, ke = min(K, kb + kc);
  const int ntiles = (ke - kb + 63) / 64;
  const rsrc ra = make_res(A, (uint64_t)M * lda * 2), rb = make_res(B, (uint64_t)N * ldb * 2);
  // this wave's DMA blocks: b = wave + 4 j; the lane's row offset (bytes, at K = kb) and K step
  uint32_t roff[PER];
  int kst[PER];
  bool isa[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int b = wave + 4 * j;
    isa[j] = b < ABLK;
    const int bb = isa[j] ? b : b - ABLK;
    kst[j] = bb & 1;
    const int row = (isa[j] ? mb : nb) + (bb >> 1) * 16 + (lane & 15);
    const int lim = isa[j] ? M : N;
    const int ld = isa[j] ? lda : ldb;
    roff[j] = row < lim ? (uint32_t)((size_t)row * ld + kb + (lane >> 4) * 8) * 2u : kOutOfRange;
  }
  f32x4m acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = f32x4m{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < NS - 1; ++t)
    if (t < ntiles) dma_tile<PER, NS, STAGE>(lds, t, wave, lane, ra, rb, roff, kst, isa, kb, ke);
  for (int t = 0; t < ntiles; ++t) {
    // this wave's blocks of tile t have landed once at most the later tiles' DMAs are pending
    // Every wave's blocks of tile t are in LDS and tile t-1's stage is free
    // once all waves pass: each waits for its own DMAs of tile t (later
    // tiles' stay in flight) and its LDS reads, then the plain s_barrier.
    // (__syncthreads would also drain every pending DMA.)
    wait_tiles<PER, NS>(min(NS - 2, ntiles - 1 - t));
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (t + NS - 1 < ntiles) dma_tile<PER, NS, STAGE>(lds, t + NS - 1, wave, lane, ra, rb, roff, kst, isa, kb, ke);
    const char* as = lds + (t % NS) * STAGE;
    const char* bs = as + ABLK * 1024;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (kb + t * 64 + ks * 32 >= ke) break;
      f16x8 a[WM], b[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i)
        a[i] = *reinterpret_cast<const f16x8*>(as + ((wr * WM + i) * 2 + ks) * 1024 + 16 * lane);
#pragma unroll
      for (int j = 0; j < WN; ++j)
        b[j] = *reinterpret_cast<const f16x8*>(bs + ((wc * WN + j) * 2 + ks) * 1024 + 16 * lane);
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
  wave_epilogue<WM, WN>(e, acc, mb + wr * WM * 16, nb + wc * WN * 16, M, N, lane);
}

// The same LDS operand-block layout, staged through registers instead of LDS
// DMA: each thread loads its 16-byte pieces of K tile t+1 (32 KS wide) into
// registers while the tile t products run, then writes them to the other of
// two LDS stages.  For the large tiles this measured faster on MI355X than
// the DMA form, best with 32-wide K tiles and three workgroups per compute
// unit (KS = 1, OCC = 3); the DMA form's deeper pipelines suit the few-row,
// weight-streaming products.
template <int BM, int BN, int KS = 2, int OCC = 1>
__global__ __launch_bounds__(256, OCC) void mp_gemm_rs(const uint16_t* __restrict__ A, int lda,
                                                       const uint16_t* __restrict__ B, int ldb, int M, int N, int K,
                                                       int kc, MpEpi e) {
  constexpr int WM = BM / 32, WN = BN / 32;
  constexpr int KT = 32 * KS;                         // K elements per tile
  constexpr int ABLK = BM / 16 * KS, BBLK = BN / 16 * KS;
  constexpr int NBLK = ABLK + BBLK, PER = NBLK / 4, STAGE = NBLK * 1024;
  static_assert(NBLK % 4 == 0, "blocks split evenly over the waves");
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  const int mb = blockIdx.y * BM, nb = blockIdx.x * BN;
  const int kb = blockIdx.z * kc, ke = min(K, kb + kc);
  const int ntiles = (ke - kb + KT - 1) / KT;
  const rsrc ra = make_res(A, (uint64_t)M * lda * 2), rb = make_res(B, (uint64_t)N * ldb * 2);
  uint32_t roff[PER];
  int kst[PER];
  bool isa[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int b = wave + 4 * j;
    isa[j] = b < ABLK;
    const int bb = isa[j] ? b : b - ABLK;
    kst[j] = bb % KS;
    const int row = (isa[j] ? mb : nb) + (bb / KS) * 16 + (lane & 15);
    const int lim = isa[j] ? M : N;
    const int ld = isa[j] ? lda : ldb;
    roff[j] = row < lim ? (uint32_t)((size_t)row * ld + kb + (lane >> 4) * 8) * 2u : kOutOfRange;
  }
  f16x8 reg[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int k0 = kst[j] * 32;
    reg[j] = ld8(isa[j] ? ra : rb, (roff[j] != kOutOfRange && kb + k0 < ke) ? roff[j] + (uint32_t)k0 * 2u : kOutOfRange);
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) *reinterpret_cast<f16x8*>(lds + (wave + 4 * j) * 1024 + 16 * lane) = reg[j];
  __syncthreads();
  f32x4m acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = f32x4m{0.f, 0.f, 0.f, 0.f};
  for (int t = 0; t < ntiles; ++t) {
    const bool next = t + 1 < ntiles;
    if (next) {
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int k0 = (t + 1) * KT + kst[j] * 32;
        reg[j] = ld8(isa[j] ? ra : rb,
                     (roff[j] != kOutOfRange && kb + k0 < ke) ? roff[j] + (uint32_t)k0 * 2u : kOutOfRange);
      }
    }
    const char* as = lds + (t & 1) * STAGE;
    const char* bs = as + ABLK * 1024;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (kb + t * KT + ks * 32 >= ke) break;
      f16x8 a[WM], b[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i)
        a[i] = *reinterpret_cast<const f16x8*>(as + ((wr * WM + i) * KS + ks) * 1024 + 16 * lane);
#pragma unroll
      for (int j = 0; j < WN; ++j)
        b[j] = *reinterpret_cast<const f16x8*>(bs + ((wc * WN + j) * KS + ks) * 1024 + 16 * lane);
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (next) {
      char* st = lds + ((t + 1) & 1) * STAGE;
#pragma unroll
      for (int j = 0; j < PER; ++j) *reinterpret_cast<f16x8*>(st + (wave + 4 * j) * 1024 + 16 * lane) = reg[j];
    }
    __syncthreads();   // tile t+1 is in LDS; tile t's stage may be overwritten
  }
  wave_epilogue<WM, WN>(e, acc, mb + wr * WM * 16, nb + wc * WN * 16, M, N, lane);
}

// The epilogue of a split-K product: the S partial slices [S][M][N] added in
// slice order, then through the product's epilogue (one thread per result,
// or per column pair in the pair modes).
__global__ __launch_bounds__(256) void mp_splitk_sum(const float* __restrict__ part, int S, int M, int N, MpEpi e) {
  const bool pair = e.mode == MP_EP_SWIGLU || e.mode == MP_EP_ROPE;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t cols = pair ? (size_t)N / 2 : (size_t)N;
  if (i >= (size_t)M * cols) return;
  const int m = (int)(i / cols), n = (int)(i - (size_t)m * cols) * (pair ? 2 : 1);
  const size_t at = (size_t)m * N + n;
  float v0 = part[at], v1 = pair ? part[at + 1] : 0.f;
  for (int z = 1; z < S; ++z) {
    v0 += part[(size_t)z * M * N + at];
    if (pair) v1 += part[(size_t)z * M * N + at + 1];
  }
  if (e.mode == MP_EP_ACCUM) {
    e.C[(size_t)m * e.ldc + n] += v0;
    return;
  }
  const float sc = e.s ? e.s[m] : 1.0f;
  if (pair) pair_store(e, m, n, v0 * sc, v1 * sc);
  else e.C[(size_t)m * e.ldc + n] = v0 * sc;
}

// DT consecutive fp16 values (DT = 2, 4 or 8) through a buffer descriptor.
template <int DT>
struct HalfRow;
template <>
struct HalfRow<8> {
  typedef _Float16 T __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ T load(rsrc r, uint32_t off) {
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  }
};
template <>
struct HalfRow<4> {
  typedef _Float16 T __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ T load(rsrc r, uint32_t off) {
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
  }
};
template <>
struct HalfRow<2> {
  typedef _Float16 T __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ T load(rsrc r, uint32_t off) {
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
  }
};

// Causal attention of queries pos0 .. pos0+n-1 of one head (blockIdx.y)
// over cache positions 0 .. pos0+n-1.  Four waves per workgroup, 16 queries
// per wave, no LDS: everything is computed transposed so that each lane owns
// one query.  For each block of 32 keys at or below the wave's last query:
//   scores S^T = K q^T on the matrix cores (A operand: key rows of the cache,
//   B operand: the wave's query rows), two 16-key tiles; lane l gets query
//   l % 16 against keys 4 (l/16) + r and 16 + 4 (l/16) + r, r = 0..3;
//   online softmax per lane (its 8 keys, then the 3 other lanes of the query);
//   O^T += V^T P^T on the matrix cores, where P^T is the lane's 8 weights in
//   fp16 as they stand (the products' K index of lane group g is keys
//   4g .. 4g+3 and 16 + 4g .. +3), and V^T's operand is built in registers:
//   lane l loads the HD/16 consecutive dims (l%16) HD/16 .. +HD/16-1 of each of
//   those 8 keys and transposes the 8 x HD/16 block, so output block t holds
//   dims c HD/16 + t for c = 0..15.
// Lane l then holds HD/16 consecutive dims per result row: o = o / sum, fp16,
// to o16 [n x q].  Query blocks run heaviest (latest) first.
template <int HD, int QG>
__global__ __launch_bounds__(256, 2) void mp_attention(const uint16_t* __restrict__ q16, int q, int n, int pos0,
                                                    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
                                                    size_t head_elems, uint16_t* __restrict__ o16) {
  constexpr int DT = HD / 16;        // dims per lane per output row; output blocks of 16 dims
  constexpr int WQ = 16 * QG;        // queries per wave: QG groups of 16 share every K/V load
  typedef HalfRow<DT> Row;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = blockIdx.y, nqb = (n + 4 * WQ - 1) / (4 * WQ);
  const int m0 = (nqb - 1 - (int)blockIdx.x) * 4 * WQ + wave * WQ;
  if (m0 >= n) return;   // the wave has no query (no barriers in this kernel)
  const int c = lane & 15, g = lane >> 4;
  const int n_keys = pos0 + n;
  const _Float16* kh = reinterpret_cast<const _Float16*>(kc) + (size_t)h * head_elems;
  const _Float16* vh = reinterpret_cast<const _Float16*>(vc) + (size_t)h * head_elems;
  const rsrc rk = make_res(kh, (uint64_t)n_keys * HD * 2), rv = make_res(vh, (uint64_t)n_keys * HD * 2);
  const rsrc rq = make_res(q16, (uint64_t)n * q * 2);
  // B operands of the score products: this lane's query row of each group, dims 32 cc + 8 g .. +7
  f16x8 qb[QG][HD / 32];
#pragma unroll
  for (int u = 0; u < QG; ++u) {
    const int m = m0 + 16 * u + c;
#pragma unroll
    for (int cc = 0; cc < HD / 32; ++cc)
      qb[u][cc] = ld8(rq, m < n ? (uint32_t)((size_t)m * q + (size_t)h * HD + 32 * cc + 8 * g) * 2u : kOutOfRange);
  }
  f32x4m acc[QG][DT];
  float mrow[QG], lsum[QG];
#pragma unroll
  for (int u = 0; u < QG; ++u) {
    mrow[u] = -INFINITY;
    lsum[u] = 0.f;
#pragma unroll
    for (int t = 0; t < DT; ++t) acc[u][t] = f32x4m{0.f, 0.f, 0.f, 0.f};
  }
  const int last = pos0 + min(m0 + WQ - 1, n - 1);   // the wave's last query position
  for (int j0 = 0; j0 <= last; j0 += 32) {
    // the 8 keys of this lane group: j0 + 4g + i (i < 4) and j0 + 16 + 4g + i - 4
    typename Row::T vrow[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = j0 + (i < 4 ? 4 * g + i : 16 + 4 * g + i - 4);
      vrow[i] = Row::load(rv, key < n_keys ? (uint32_t)(key * HD + c * DT) * 2u : kOutOfRange);
    }
    f16x8 ka[HD / 32], kb[HD / 32];
#pragma unroll
    for (int cc = 0; cc < HD / 32; ++cc) {
      const int ja = j0 + c, jb = j0 + 16 + c;
      ka[cc] = ld8(rk, ja < n_keys ? (uint32_t)(ja * HD + 32 * cc + 8 * g) * 2u : kOutOfRange);
      kb[cc] = ld8(rk, jb < n_keys ? (uint32_t)(jb * HD + 32 * cc + 8 * g) * 2u : kOutOfRange);
    }
    // V^T operands, output block t = dims c DT + t (shared by the query groups)
    f16x8 va[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int i = 0; i < 8; ++i) va[t][i] = vrow[i][t];
#pragma unroll
    for (int u = 0; u < QG; ++u) {
      if (j0 > pos0 + m0 + 16 * u + 15) continue;   // every key of the block is past this group (wave-uniform)
      // scores S^T = K q^T: s0[r] for key j0 + 4g + r, s1[r] for key j0 + 16 + 4g + r
      f32x4m s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cc = 0; cc < HD / 32; ++cc) {
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[cc], qb[u][cc], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(kb[cc], qb[u][cc], s1, 0, 0, 0);
      }
      // online softmax of the lane's query over the 32 keys
      const int qi = pos0 + m0 + 16 * u + c;
      float p[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = (j0 + 4 * g + r <= qi) ? s0[r] : -INFINITY;
        p[4 + r] = (j0 + 16 + 4 * g + r <= qi) ? s1[r] : -INFINITY;
      }
      float mx = p[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, p[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // key 0 is at or below every query, so the max is finite from the first block on
      const float mn = fmaxf(mrow[u], mx);
      const float alpha = expf(mrow[u] - mn);
      f16x8 pb;
      float rs = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float ev = expf(p[i] - mn);
        rs += ev;
        pb[i] = (_Float16)ev;
      }
      rs += __shfl_xor(rs, 16, 64);
      rs += __shfl_xor(rs, 32, 64);
      lsum[u] = lsum[u] * alpha + rs;
      mrow[u] = mn;
      // O^T += V^T P^T
#pragma unroll
      for (int t = 0; t < DT; ++t)
        acc[u][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[t], pb, acc[u][t] * alpha, 0, 0, 0);
    }
  }
#pragma unroll
  for (int u = 0; u < QG; ++u) {
    const int m = m0 + 16 * u + c;
    if (m >= n) continue;
    const float inv = 1.0f / lsum[u];
    _Float16* orow = reinterpret_cast<_Float16*>(o16) + (size_t)m * q + (size_t)h * HD;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      typename Row::T o;
#pragma unroll
      for (int t = 0; t < DT; ++t) o[t] = (_Float16)(acc[u][t][r] * inv);
      *reinterpret_cast<typename Row::T*>(orow + (4 * g + r) * DT) = o;
    }
  }
}

// The greedy token of one logits row (lowest index on ties): one workgroup,
// each thread over a strided share in index order, then a fixed-order tree.
__global__ __launch_bounds__(1024) void mp_argmax(const float* __restrict__ logits, int V, int* __restrict__ tok_out,
                                                  int* __restrict__ tok_cur) {
  __shared__ float bv[1024];
  __shared__ int bi[1024];
  const int tid = threadIdx.x;
  float best = -INFINITY;
  int idx = 0x7fffffff;
  for (int i = tid; i < V; i += 1024) {
    const float v = logits[i];
    if (v > best) {
      best = v;
      idx = i;
    }
  }
  bv[tid] = best;
  bi[tid] = idx;
  __syncthreads();
  for (int w = 512; w >= 1; w >>= 1) {
    if (tid < w) {
      const float ov = bv[tid + w];
      const int oi = bi[tid + w];
      if (ov > bv[tid] || (ov == bv[tid] && oi < bi[tid])) {
        bv[tid] = ov;
        bi[tid] = oi;
      }
    }
    __syncthreads();
  }
  if (tid == 0) {
    const int t = bi[0] == 0x7fffffff ? 0 : bi[0];
    *tok_out = t;
    *tok_cur = t;
  }
}

// Tile shapes (index = MpGemm::shape): register-staged 128 x 128 and
// 128 x 64 tiles for many rows; LDS-DMA 64 x 64, 128 x 64 and 64 x 32 tiles
// with four K tiles in flight for up to 128 rows, where the product streams
// the weights; the register-direct 16 x 64 tile for one to 16 rows.
constexpr int kShapeBM[kMpShapes] = {128, 128, 64, 128, 64, 16};
constexpr int kShapeBN[kMpShapes] = {128, 64, 64, 64, 32, 64};

template <int BM, int BN, int NS>
constexpr int lds_bytes() { return NS * (BM / 16 * 2 + BN / 16 * 2) * 1024; }

template <int BM, int BN, int NS>
hipError_t prepare_lds() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&mp_gemm_lds<BM, BN, NS>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes<BM, BN, NS>());
}
// register-staged tiles: 32-wide K tiles in two LDS stages, three workgroups per compute unit
template <int BM, int BN>
constexpr int rs_lds_bytes() { return 2 * (BM / 16 + BN / 16) * 1024; }
template <int BM, int BN>
hipError_t prepare_rs() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&mp_gemm_rs<BM, BN, 1, 3>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, rs_lds_bytes<BM, BN>());
}

template <int BM, int BN, int NS>
void gemm_lds_as(const MpGemm& g, const MpEpi& e, dim3 grid, hipStream_t st) {
  constexpr int lds = lds_bytes<BM, BN, NS>();
  hipLaunchKernelGGL((mp_gemm_lds<BM, BN, NS>), grid, dim3(256), lds, st, g.A, g.lda, g.B, g.ldb, g.M, g.N, g.K,
                     g.kc, e);
}

template <int BM, int BN>
void gemm_rs_as(const MpGemm& g, const MpEpi& e, dim3 grid, hipStream_t st) {
  constexpr int lds = rs_lds_bytes<BM, BN>();
  hipLaunchKernelGGL((mp_gemm_rs<BM, BN, 1, 3>), grid, dim3(256), lds, st, g.A, g.lda, g.B, g.ldb, g.M, g.N, g.K,
                     g.kc, e);
}

template <int WM, int WN, int WR>
void gemm_as(const MpGemm& g, const MpEpi& e, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((mp_gemm<WM, WN, WR>), grid, dim3(256), 0, st, g.A, g.lda, g.B, g.ldb, g.M, g.N, g.K, g.kc, e);
}

}  // namespace

// Raise the dynamic-LDS limit of the LDS-staged products (once per process).
int mp_prepare() {
  hipError_t e = prepare_rs<128, 128>();
  if (e == hipSuccess) e = prepare_rs<128, 64>();
  if (e == hipSuccess) e = prepare_lds<64, 64, 4>();
  if (e == hipSuccess) e = prepare_lds<128, 64, 4>();
  if (e == hipSuccess) e = prepare_lds<64, 32, 4>();
  return (int)e;
}

// Tile shape and K split of a product.  One to 16 rows: the register-direct
// tile.  Up to 512 rows: 64 x 64 LDS-DMA tiles (128 x 64 above 64 rows for
// the widest and the deepest products).  More rows: the register-staged
// 128 x 128 tile.  Then the K range is split (up to 8 ways, each split 4 K
// steps or more, partials within part_floats) until about 150 workgroups
// run (200 for the register-staged tile).  The choices follow timings of the
// dense2b products on MI355X at 1 to 3968 rows.
void mp_plan(int M, int N, int K, size_t part_floats, int* shape, int* S, int* kc) {
  auto count = [&](int t) {
    return (long long)((M + kShapeBM[t] - 1) / kShapeBM[t]) * ((N + kShapeBN[t] - 1) / kShapeBN[t]);
  };
  int pick;
  if (M <= 16) pick = 5;
  else if (M <= 512) pick = (M > 64 && (N >= 8192 || K >= 4096)) ? 3 : 2;
  else pick = 0;
  int s = 1;
  const long long c = count(pick);
  const long long want = M <= 512 ? 150 : 200;
  while (s < 8 && c * s < want && K / (32 * 2 * s) >= 4 && (size_t)(2 * s) * M * N <= part_floats) s *= 2;
  const int steps = (K / 32 + s - 1) / s;   // K steps per split
  *shape = pick;
  *S = (K / 32 + steps - 1) / steps;
  *kc = steps * 32;
}

// Host-side launches of the matrix prefill (each returns a hipError_t value).
int mp_launch_embed(const uint16_t* E, const int* tok, int n, int d, float* x, void* stream) {
  hipLaunchKernelGGL(mp_embed, dim3(n), dim3(256), 0, (hipStream_t)stream, E, tok, d, x);
  return (int)hipGetLastError();
}
int mp_launch_norm(const float* x, const float* g, int n, int d, float eps, uint16_t* h, float* s, void* stream) {
  hipLaunchKernelGGL(mp_norm, dim3(n), dim3(256), 0, (hipStream_t)stream, x, g, d, eps, h, s);
  return (int)hipGetLastError();
}
int mp_launch_gemm(const MpGemm& g, void* stream) {
  const bool pair = g.epi.mode == MP_EP_SWIGLU || g.epi.mode == MP_EP_ROPE;
  if (g.K < 32 || g.K % 32 || g.M < 1 || g.N < 1 || g.shape < 0 || g.shape >= kMpShapes || g.S < 1 || g.kc < 32 ||
      g.kc % 32 || (long long)g.S * g.kc < g.K || (long long)(g.S - 1) * g.kc >= g.K || (g.S > 1 && !g.part) ||
      g.epi.mode < MP_EP_SCALE || g.epi.mode > MP_EP_ROPE || g.epi.mode == MP_EP_PART || (pair && g.N % 2) ||
      (g.epi.mode == MP_EP_ROPE && (g.N != 3 * g.epi.q || g.epi.q % g.epi.hd || g.epi.hd % 2)))
    return (int)hipErrorInvalidValue;
  const dim3 grid((g.N + kShapeBN[g.shape] - 1) / kShapeBN[g.shape], (g.M + kShapeBM[g.shape] - 1) / kShapeBM[g.shape],
                  g.S);
  const hipStream_t st = (hipStream_t)stream;
  MpEpi e = g.epi;
  if (g.S > 1) {   // the product writes its partial sums; the sum kernel applies the epilogue
    e.mode = MP_EP_PART;
    e.C = g.part;
  }
  switch (g.shape) {
    case 0: gemm_rs_as<128, 128>(g, e, grid, st); break;
    case 1: gemm_rs_as<128, 64>(g, e, grid, st); break;
    case 2: gemm_lds_as<64, 64, 4>(g, e, grid, st); break;
    case 3: gemm_lds_as<128, 64, 4>(g, e, grid, st); break;
    case 4: gemm_lds_as<64, 32, 4>(g, e, grid, st); break;
    default: gemm_as<1, 1, 1>(g, e, grid, st); break;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || g.S == 1) return (int)err;
  const size_t total = (size_t)g.M * (pair ? g.N / 2 : g.N);
  hipLaunchKernelGGL(mp_splitk_sum, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, g.part, g.S, g.M, g.N,
                     g.epi);
  return (int)hipGetLastError();
}
int mp_launch_attention(const uint16_t* q16, int q, int n, int pos0, int H, int hd, const uint16_t* kc,
                        const uint16_t* vc, size_t head_elems, uint16_t* o16, void* stream) {
  constexpr int QG = 2;   // query groups of 16 per wave
  const dim3 grid((n + 64 * QG - 1) / (64 * QG), H);
  const hipStream_t st = (hipStream_t)stream;
  switch (hd) {
    case 32: hipLaunchKernelGGL((mp_attention<32, QG>), grid, dim3(256), 0, st, q16, q, n, pos0, kc, vc, head_elems, o16); break;
    case 64: hipLaunchKernelGGL((mp_attention<64, QG>), grid, dim3(256), 0, st, q16, q, n, pos0, kc, vc, head_elems, o16); break;
    case 128: hipLaunchKernelGGL((mp_attention<128, QG>), grid, dim3(256), 0, st, q16, q, n, pos0, kc, vc, head_elems, o16); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}
int mp_launch_argmax(const float* logits, int V, int* tok_out, int* tok_cur, void* stream) {
  hipLaunchKernelGGL(mp_argmax, dim3(1), dim3(1024), 0, (hipStream_t)stream, logits, V, tok_out, tok_cur);
  return (int)hipGetLastError();
}

}  // namespace decmono
