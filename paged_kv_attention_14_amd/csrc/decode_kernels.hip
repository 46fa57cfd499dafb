// Paged-KV split-K decode kernels for gfx950 (MI355X).
//
// One workgroup handles one (sequence b, kv head hk, split s). Its NW waves
// take 32-token tiles of the split round-robin; each wave keeps its own
// online-softmax state and the waves merge through LDS at the end. The split
// partition, the online softmax and the partial (O, LSE) combine follow the
// split-K FlashAttention organisation of "Implementing a High-Performance
// Custom Diffusion Attention Kernel with FlyDSL" (introduction item 3; "Debug
// Systematically" for the LSE intermediate) and the decode + reduce kernel
// pair of "[ROCm] Add FlyDSL paged-attention decode backend (dense + fp8) with
// benchmark" (Kernels).
//
// Matrix-core mapping (v_mfma_f32_16x16x32_{bf16,f16}, wave64):
//  * The g*Tq query rows that share kv head hk are packed into the 16-wide N
//    side of the tile (head packing, same pull request, Kernels), zero-padded.
//  * QK^T is computed operand-swapped: A = K (M = 16 tokens), B = Q (N = rows),
//    as the FlyDSL blog recommends ("Match MFMA Operands to the Desired
//    Fragment Layout"). Lane l then holds scores of row l%16 for tokens
//    4*(l/16)+i, i = 0..3, of each 16-token subtile.
//  * P.V is computed as O^T = V^T P^T with A = V^T (M = 16 head dims) and
//    B = P^T. Its K side is the 32 tokens of the tile. A lane's eight B
//    elements are exactly the eight scores it already holds (subtile 0 then
//    subtile 1), so P never leaves registers; V^T is read from LDS in the
//    matching token order.
//  * The contraction index of both products may be permuted freely as long as
//    both operands use the same permutation, so every operand is loaded in
//    the order that makes its memory access contiguous.
//
// K rows are loaded straight from HBM into the A operand (16 contiguous bytes
// per lane). V rows are loaded with full-row coalescing and staged in a
// per-wave LDS tile, then read back transposed. fp8 e4m3fn codes are decoded
// to the 16-bit MFMA type on the way into the operands (exact: every e4m3fn
// value is representable in bf16 and f16); the per-token K scale multiplies
// the score, the per-token V scale multiplies the probability before the
// cast (the softmax sum uses the unscaled probability).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_launch.h"

namespace pdk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Vec8;
template <> struct Vec8<__bf16> { typedef bf16x8 type; };
template <> struct Vec8<_Float16> { typedef f16x8 type; };

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr int kTile = 32;      // tokens per wave iteration (K side of P.V)
constexpr float kLn2 = 0.69314718055994530942f;

// Decode 8 e4m3fn codes (two little-endian dwords) to 8 elements of T.
template <typename T>
__device__ __forceinline__ typename Vec8<T>::type decode8(uint32_t lo, uint32_t hi) {
  typename Vec8<T>::type r;
  f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false);
  f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);
  f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
  f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
  r[0] = (T)a[0]; r[1] = (T)a[1]; r[2] = (T)b[0]; r[3] = (T)b[1];
  r[4] = (T)c[0]; r[5] = (T)c[1]; r[6] = (T)d[0]; r[7] = (T)d[1];
  return r;
}

template <typename T>
__device__ __forceinline__ typename Vec8<T>::type as_vec8(u32x4 x) {
  return __builtin_bit_cast(typename Vec8<T>::type, x);
}

// Element-row index of (token t, kv head hk) in the extended token space of
// sequence b: tokens below ctx are paged (row of the page pool), tokens from
// ctx on are scratch (row of the scratch area). Branch-free, so the caller
// selects the base pointer with a plain conditional move.
__device__ __forceinline__ int64_t kv_row(int t, int ctx, int page, int log2bs, int Hkv,
                                          int hk, int b, int stok) {
  const int64_t paged = ((((int64_t)page << log2bs) + (t & ((1 << log2bs) - 1))) * Hkv) + hk;
  const int64_t scratch = (((int64_t)b * stok + (t - ctx)) * Hkv) + hk;
  return (t < ctx) ? paged : scratch;
}

// Registers of one 32-token tile in flight.
template <bool FP8, int KLOADS, int VLOADS>
struct TileRegs {
  u32x4 k[KLOADS];
  u32x4 v[VLOADS];
  float ks[8];  // fp8: K scales of the lane's eight score tokens
  float vs[8];  // fp8: V scales of the same tokens
};

template <typename QT, bool FP8, int D, int NW>
__global__ __launch_bounds__(NW * 64, (D >= 256) ? 1 : 2) void paged_decode_kernel(DecodeParams p) {
  typedef typename Vec8<QT>::type vec8;
  constexpr int ESZ = FP8 ? 1 : 2;           // bytes per KV element
  constexpr int ROWB = D * ESZ;              // bytes of one (token, kv head) row
  constexpr int CPR = ROWB / 16;             // 16-byte chunks per row
  constexpr int KSTEPS = D / 32;             // MFMA k-steps over the head dim
  constexpr int DT = D / 16;                 // 16-wide head-dim tiles of O
  constexpr int KL_PER_SUB = FP8 ? KSTEPS / 2 : KSTEPS;  // 16-B K loads per subtile
  constexpr int KLOADS = 2 * KL_PER_SUB;
  constexpr int VLOADS = kTile * CPR / 64;
  constexpr int PITCH = ROWB + 16;           // LDS row pitch of the staged V tile
  constexpr int STAGE = kTile * PITCH;       // bytes per wave
  constexpr int MPITCH = D + 4;              // floats per row of the merge buffer
  constexpr int MERGE = NW * 16 * MPITCH * 4;
  constexpr int LDSB = (NW * STAGE > MERGE) ? NW * STAGE : MERGE;
  static_assert(VLOADS * 64 == kTile * CPR, "V tile must split evenly over a wave");

  __shared__ __attribute__((aligned(16))) char lds[LDSB];
  __shared__ float ml[2][NW][16];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lr = lane & 15;   // row (N) / token (M) / head dim (M) index within 16
  const int lg = lane >> 4;   // 0..3: which 8-element slice of the K side

  const int S = p.S;
  const int s = blockIdx.x % S;
  const int bh = blockIdx.x / S;
  const int hk = bh % p.Hkv;
  const int b = bh / p.Hkv;

  const int bs = 1 << p.log2bs;
  const int ctx = p.ctx[b];
  const int npages = (ctx + bs - 1) >> p.log2bs;
  const int pps = (npages + S - 1) / S;
  const int p0 = min(s * pps, npages);
  const int p1 = min((s + 1) * pps, npages);
  const int lo = min(p0 << p.log2bs, ctx);
  const int hi = min(p1 << p.log2bs, ctx);
  const int end = hi + ((s == S - 1) ? p.stok : 0);
  const int rows = p.rows;

  // Output row r <-> (query token r / g, q head hk * g + r % g).
  auto out_row = [&](int r) -> int64_t {
    const int tq = r / p.g;
    const int h = hk * p.g + (r % p.g);
    return ((int64_t)b * p.Tq + tq) * p.Hq + h;
  };

  if (lo >= end) {
    // Empty split: O_s = 0, LSE_s = -inf (or the final output when S == 1).
    for (int e = threadIdx.x; e < rows * D; e += NW * 64) {
      const int r = e / D, d = e % D;
      if (S == 1) ((QT*)p.out)[out_row(r) * D + d] = (QT)0.0f;
      else p.opart[(out_row(r) * S + s) * D + d] = 0.0f;
    }
    if (threadIdx.x < rows) {
      if (S == 1) { if (p.lse) p.lse[out_row(threadIdx.x)] = -__builtin_inff(); }
      else p.lpart[out_row(threadIdx.x) * S + s] = -__builtin_inff();
    }
    return;
  }

  const int32_t* bt_row = p.bt + (int64_t)b * p.bt_stride;
  const char* const kpool = (const char*)p.k;
  const char* const vpool = (const char*)p.v;
  const char* const kscr = (const char*)p.sk;
  const char* const vscr = (const char*)p.sv;
  const float* const kscale = p.ks;
  const float* const vscale = p.vs;
  const int log2bs = p.log2bs;
  const int Hkv = p.Hkv;
  const int stok = p.stok;

  // Query operand: lane (row lr, slice lg) holds Q[row][dchunk(step, lg) .. +8].
  // dchunk matches the K loads: dense 32*step + 8*lg; fp8 64*(step/2) + 16*lg + 8*(step%2).
  vec8 qop[KSTEPS];
  {
    const bool live = lr < rows;
    const QT* qrow = (const QT*)p.q + (live ? out_row(lr) : 0) * D;
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st) {
      const int dc = FP8 ? (64 * (st / 2) + 16 * lg + 8 * (st % 2)) : (32 * st + 8 * lg);
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (live) raw = *(const u32x4*)(qrow + dc);
      qop[st] = as_vec8<QT>(raw);
    }
  }

  const int ntiles = (end - lo + kTile - 1) / kTile;
  const int my_tiles = (ntiles > wave) ? (ntiles - wave + NW - 1) / NW : 0;

  f32x4 acc[DT];
#pragma unroll
  for (int n = 0; n < DT; ++n) acc[n] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();
  float l_run = 0.f;

  char* stage = lds + wave * STAGE;
  const int ctx_pages = npages;

  // Block-table entries of one tile: lane L < 32 holds the physical page of
  // logical page (tile_start >> log2bs) + L when that page is in the context.
  auto load_pages = [&](int j) -> int {
    const int ts = lo + (wave + NW * j) * kTile;
    const int first = ts >> log2bs;
    const int last = (min(ts + kTile, end) - 1) >> log2bs;
    const int pi = first + lane;
    int pg = 0;
    if (lane < 32 && pi <= last && pi < ctx_pages) pg = bt_row[pi];
    return pg;
  };

  auto load_tile = [&](int j, int pv, TileRegs<FP8, KLOADS, VLOADS>& t) {
    const int ts = lo + (wave + NW * j) * kTile;
    const int first = ts >> log2bs;
    // K: subtile u, lane token ts + 16u + lr, chunks KL_PER_SUB along the row.
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int tok = min(ts + 16 * u + lr, end - 1);
      const int page = __shfl(pv, (tok >> log2bs) - first);
      const char* kr = ((tok < ctx) ? kpool : kscr) +
                       kv_row(tok, ctx, page, log2bs, Hkv, hk, b, stok) * ROWB;
#pragma unroll
      for (int c = 0; c < KL_PER_SUB; ++c)
        t.k[u * KL_PER_SUB + c] = *(const u32x4*)(kr + 64 * c + 16 * lg);
    }
    // V: chunk q = i*64 + lane covers token q / CPR, bytes (q % CPR) * 16.
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int q = i * 64 + lane;
      const int tok = min(ts + q / CPR, end - 1);
      const int page = __shfl(pv, (tok >> log2bs) - first);
      const char* vr = ((tok < ctx) ? vpool : vscr) +
                       kv_row(tok, ctx, page, log2bs, Hkv, hk, b, stok) * ROWB;
      t.v[i] = *(const u32x4*)(vr + (q % CPR) * 16);
    }
    if constexpr (FP8) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = min(ts + 16 * u + 4 * lg + i, end - 1);
          const int page = __shfl(pv, (tok >> log2bs) - first);
          const int64_t idx = kv_row(tok, ctx, page, log2bs, Hkv, hk, b, stok);
          t.ks[u * 4 + i] = kscale[idx];
          t.vs[u * 4 + i] = vscale[idx];
        }
      }
    }
  };

  auto compute_tile = [&](int j, const TileRegs<FP8, KLOADS, VLOADS>& t) {
    const int ts = lo + (wave + NW * j) * kTile;
    const int nvalid = min(kTile, end - ts);

    // Stage V rows in LDS (natural layout, padded pitch).
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int q = i * 64 + lane;
      *(u32x4*)(stage + (q / CPR) * PITCH + (q % CPR) * 16) = t.v[i];
    }

    // Scores S[token][row] for the two 16-token subtiles.
    f32x4 sc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < KSTEPS; ++st) {
        vec8 kop;
        if constexpr (FP8) {
          const u32x4 w = t.k[u * KL_PER_SUB + st / 2];
          kop = (st % 2) ? decode8<QT>(w[2], w[3]) : decode8<QT>(w[0], w[1]);
        } else {
          kop = as_vec8<QT>(t.k[u * KL_PER_SUB + st]);
        }
        a = mfma16x16x32(kop, qop[st], a);
      }
      sc[u] = a;
    }

    float sv[8];
    float mt = -__builtin_inff();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tl = 16 * u + 4 * lg + i;
        float x = sc[u][i] * p.scale_log2;
        if constexpr (FP8) x *= t.ks[u * 4 + i];
        x = (tl < nvalid) ? x : -__builtin_inff();
        sv[u * 4 + i] = x;
        mt = fmaxf(mt, x);
      }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = fast_exp2(m_run - m_new);
    float lsum = 0.f;
    vec8 pop;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pe = fast_exp2(sv[e] - m_new);
      lsum += pe;
      float pw = pe;
      if constexpr (FP8) pw *= t.vs[e];
      pop[e] = (QT)pw;
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;

    __builtin_amdgcn_wave_barrier();
    // V^T operand for head-dim tile n: lane (lr, lg) needs V[tok(lg, e)][16n + lr]
    // with tok(lg, e) = 4lg + e (e < 4) or 16 + 4lg + (e - 4) (e >= 4).
#pragma unroll
    for (int n = 0; n < DT; ++n) {
      const int dcol = 16 * n + lr;
      vec8 vop;
      if constexpr (FP8) {
        uint32_t w0 = 0, w1 = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int tk = (e < 4) ? (4 * lg + e) : (16 + 4 * lg + e - 4);
          const uint32_t byte = *(const uint8_t*)(stage + tk * PITCH + dcol);
          if (e < 4) w0 |= byte << (8 * e);
          else w1 |= byte << (8 * (e - 4));
        }
        vop = decode8<QT>(w0, w1);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int tk = (e < 4) ? (4 * lg + e) : (16 + 4 * lg + e - 4);
          vop[e] = *(const QT*)(stage + tk * PITCH + dcol * 2);
        }
      }
      f32x4 o = acc[n] * alpha;
      acc[n] = mfma16x16x32(vop, pop, o);
    }
    __builtin_amdgcn_wave_barrier();
  };

  // Software pipeline: while tile j is computed, the data of tile j + 1 and the
  // block-table entries of tile j + 2 are in flight. Indices past the last tile
  // are clamped to it (a harmless reload), so every iteration issues the same
  // loads and the memory counters stay in program order.
  if (my_tiles > 0) {
    const int last = my_tiles - 1;
    TileRegs<FP8, KLOADS, VLOADS> ta, tb;
    int pv_next = load_pages(min(1, last));
    {
      const int pv0 = load_pages(0);
      load_tile(0, pv0, ta);
    }
    for (int j = 0; j < my_tiles; j += 2) {
      int pv_after = load_pages(min(j + 2, last));
      load_tile(min(j + 1, last), pv_next, tb);
      compute_tile(j, ta);
      pv_next = pv_after;
      if (j + 1 > last) break;
      pv_after = load_pages(min(j + 3, last));
      load_tile(min(j + 2, last), pv_next, ta);
      compute_tile(j + 1, tb);
      pv_next = pv_after;
    }
  }

  // Finish this wave: the four lanes of a row share m_run; sum their l.
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (lg == 0) {
    ml[0][wave][lr] = m_run;
    ml[1][wave][lr] = l_run;
  }
  __syncthreads();

  // Merge the waves: M = max m_w, L = sum l_w 2^(m_w - M), weight_w = 2^(m_w - M) / L.
  float M = -__builtin_inff();
#pragma unroll
  for (int w = 0; w < NW; ++w) M = fmaxf(M, ml[0][w][lr]);
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) L += ml[1][w][lr] * fast_exp2(ml[0][w][lr] - M);
  const float wgt = fast_exp2(m_run - M) / L;

  float* mrg = (float*)lds;
#pragma unroll
  for (int n = 0; n < DT; ++n) {
    f32x4 o = acc[n] * wgt;
    *(f32x4*)(mrg + (wave * 16 + lr) * MPITCH + 16 * n + 4 * lg) = o;
  }
  __syncthreads();

  for (int e = threadIdx.x; e < rows * (D / 4); e += NW * 64) {
    const int r = e / (D / 4);
    const int d4 = (e % (D / 4)) * 4;
    f32x4 o = *(const f32x4*)(mrg + r * MPITCH + d4);
#pragma unroll
    for (int w = 1; w < NW; ++w) o += *(const f32x4*)(mrg + (w * 16 + r) * MPITCH + d4);
    const int64_t orow = out_row(r);
    if (S == 1) {
      QT* dst = (QT*)p.out + orow * D + d4;
      dst[0] = (QT)o[0]; dst[1] = (QT)o[1]; dst[2] = (QT)o[2]; dst[3] = (QT)o[3];
    } else {
      *(f32x4*)(p.opart + (orow * S + s) * D + d4) = o;
    }
  }
  if (threadIdx.x < rows) {
    const int r = threadIdx.x;
    float Mr = -__builtin_inff();
    for (int w = 0; w < NW; ++w) Mr = fmaxf(Mr, ml[0][w][r]);
    float Lr = 0.f;
    for (int w = 0; w < NW; ++w) Lr += ml[1][w][r] * fast_exp2(ml[0][w][r] - Mr);
    const float lse = (Mr + __builtin_amdgcn_logf(Lr)) * kLn2;
    if (S == 1) { if (p.lse) p.lse[out_row(r)] = lse; }
    else p.lpart[out_row(r) * S + s] = lse;
  }
}

// Split-K combine: one 64-lane workgroup per (b, t, h).
template <typename QT, int D>
__global__ __launch_bounds__(64) void paged_decode_reduce_kernel(ReduceParams p) {
  const int64_t row = blockIdx.x;
  const int S = p.S;
  const float* lp = p.lpart + row * S;
  float M = -__builtin_inff();
  for (int s = 0; s < S; ++s) M = fmaxf(M, lp[s]);
  QT* out = (QT*)p.out + row * D;
  if (M == -__builtin_inff()) {
    for (int d = threadIdx.x; d < D; d += 64) out[d] = (QT)0.0f;
    if (threadIdx.x == 0 && p.lse) p.lse[row] = -__builtin_inff();
    return;
  }
  float wsum = 0.f;
  for (int s = 0; s < S; ++s) wsum += __expf(lp[s] - M);
  const float inv = 1.0f / wsum;
  for (int d = threadIdx.x; d < D; d += 64) {
    float o = 0.f;
    for (int s = 0; s < S; ++s) o += __expf(lp[s] - M) * p.opart[(row * S + s) * D + d];
    out[d] = (QT)(o * inv);
  }
  if (threadIdx.x == 0 && p.lse) p.lse[row] = M + __logf(wsum);
}

// ---------------------------------------------------------------------------
// Launch table.

template <typename QT, bool FP8, int D>
static hipError_t launch_decode_t(const DecodeParams& p, int grid, hipStream_t stream) {
  constexpr int NW = 4;
  hipLaunchKernelGGL((paged_decode_kernel<QT, FP8, D, NW>), dim3(grid), dim3(NW * 64), 0,
                     stream, p);
  return hipGetLastError();
}

template <typename QT>
static hipError_t launch_decode_q(const DecodeParams& p, bool fp8, int D, int grid,
                                  hipStream_t stream) {
  if (fp8) {
    switch (D) {
      case 64: return launch_decode_t<QT, true, 64>(p, grid, stream);
      case 128: return launch_decode_t<QT, true, 128>(p, grid, stream);
      case 256: return launch_decode_t<QT, true, 256>(p, grid, stream);
    }
  } else {
    switch (D) {
      case 64: return launch_decode_t<QT, false, 64>(p, grid, stream);
      case 128: return launch_decode_t<QT, false, 128>(p, grid, stream);
      case 256: return launch_decode_t<QT, false, 256>(p, grid, stream);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeParams& p, bool q_f16, bool kv_fp8, int head_dim,
                         int grid, hipStream_t stream) {
  return q_f16 ? launch_decode_q<_Float16>(p, kv_fp8, head_dim, grid, stream)
               : launch_decode_q<__bf16>(p, kv_fp8, head_dim, grid, stream);
}

template <typename QT>
static hipError_t launch_reduce_q(const ReduceParams& p, int D, int grid, hipStream_t stream) {
  switch (D) {
    case 64:
      hipLaunchKernelGGL((paged_decode_reduce_kernel<QT, 64>), dim3(grid), dim3(64), 0, stream, p);
      break;
    case 128:
      hipLaunchKernelGGL((paged_decode_reduce_kernel<QT, 128>), dim3(grid), dim3(64), 0, stream, p);
      break;
    case 256:
      hipLaunchKernelGGL((paged_decode_reduce_kernel<QT, 256>), dim3(grid), dim3(64), 0, stream, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_reduce(const ReduceParams& p, bool q_f16, int head_dim, int grid,
                         hipStream_t stream) {
  return q_f16 ? launch_reduce_q<_Float16>(p, head_dim, grid, stream)
               : launch_reduce_q<__bf16>(p, head_dim, grid, stream);
}

}  // namespace pdk
