// KV-cache write for the paged decode library, gfx950 (MI355X).
//
// New tokens' K and V rows are written into the page slots the caller names
// (slot = page * block_size + offset; a negative slot, or one at or past the
// pool capacity when the caller gives it, skips the token). For
// an e4m3fn cache each (token, kv head) row is quantised on the way in, with
// one symmetric scale per row: the scale is set when the cache is written,
// not in every decode call ("[ROCm] Add FlyDSL paged-attention decode backend
// (dense + fp8) with benchmark", review thread; the decode kernel reads
// e4m3fn codes with a per-token scale, Kernels).
//
// fp8 rows: absmax over the D values, scale = absmax / 448 and y = x / scale
// (both correctly rounded in single precision; the quotients from one
// reciprocal per row and a correction step), codes = e4m3fn of
// clamp(y, -448, 448) rounded to nearest even by the gfx950 packed
// conversion; a zero row gets scale 0 and codes 0. With f16 scale storage
// the scale is first rounded to f16 (nearest even, at most the largest
// finite f16) and the rounded value both divides x and is stored; a row whose
// rounded scale is 0 gets codes 0.
//
// Each wave handles a few (token, kv head) rows; 16 lanes hold a row, D/16
// consecutive values each.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_launch.h"

namespace pdk {

namespace {

constexpr float kE4m3Max = 448.0f;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// A lane's E consecutive 16-bit values of a row (E = 4, 8 or 16), moved with
// 8- or 16-byte accesses.
template <int E> struct Raw16;
template <> struct Raw16<4> {
  u32x2 w;
  __device__ __forceinline__ void load(const void* p) { w = *(const u32x2*)p; }
  __device__ __forceinline__ void store(void* p) const { *(u32x2*)p = w; }
  __device__ __forceinline__ uint32_t word(int i) const { return w[i]; }
};
template <> struct Raw16<8> {
  u32x4 w;
  __device__ __forceinline__ void load(const void* p) { w = *(const u32x4*)p; }
  __device__ __forceinline__ void store(void* p) const { *(u32x4*)p = w; }
  __device__ __forceinline__ uint32_t word(int i) const { return w[i]; }
};
template <> struct Raw16<16> {
  u32x4 w[2];
  __device__ __forceinline__ void load(const void* p) {
    w[0] = ((const u32x4*)p)[0];
    w[1] = ((const u32x4*)p)[1];
  }
  __device__ __forceinline__ void store(void* p) const {
    ((u32x4*)p)[0] = w[0];
    ((u32x4*)p)[1] = w[1];
  }
  __device__ __forceinline__ uint32_t word(int i) const { return w[i >> 2][i & 3]; }
};

// Value h (0: low half, 1: high half) of a word of two bf16 / f16 values.
template <typename QT>
__device__ __forceinline__ float half_to_f32(uint32_t w, int h) {
  const uint32_t b = h ? (w >> 16) : (w & 0xffffu);
  if constexpr (__is_same(QT, __bf16))
    return __builtin_bit_cast(float, b << 16);
  else
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// Maximum over the 16 lanes of a row of the wave (every lane of the row gets
// it): DPP quad swaps, then the half-row and row mirrors.
template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
  const int o = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false);
  return fmaxf(v, __builtin_bit_cast(float, o));
}
__device__ __forceinline__ float row16_max(float v) {
  v = dpp_max<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v = dpp_max<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v = dpp_max<0x141>(v);  // row_half_mirror
  v = dpp_max<0x140>(v);  // row_mirror
  return v;
}

// Quantise one row, held by 16 lanes (this lane's E values in x), and store
// this lane's E codes and, from the row's first lane, the scale.
template <int E>
__device__ __forceinline__ void put_fp8_row(const float* x, uint8_t* codes, void* scale_out,
                                            bool f16, bool first) {
  float am = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) am = fmaxf(am, fabsf(x[e]));
  am = row16_max(am);
  float scale = __fdiv_rn(am, kE4m3Max);
  if (f16) scale = (float)(_Float16)fminf(scale, 65504.0f);
  // x / scale, correctly rounded, from one reciprocal per row: with
  // r = RN(1 / scale), q = RN(x * r) and the residual e = fma(-q, scale, x),
  // fma(e, r, q) is the correctly rounded quotient (Markstein's correction
  // step). Checked exhaustively against IEEE division for every bf16 x and
  // every f32 and f16 scale this write can produce down to 2^-64, over the
  // quotients in [2^-11, 448 (1 + 2^-8)] where the e4m3 code depends on the
  // exact rounding (smaller quotients give code 0, larger ones clamp);
  // negative x by symmetry; zero, infinite and NaN x give what the division
  // gives. Rows with a smaller or non-finite scale divide directly.
  const bool recip = scale >= 0x1p-64f && scale <= 3.0e38f;
  float y[E];
  if (recip) {
    const float r = __fdiv_rn(1.0f, scale);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float q = __fmul_rn(x[e], r);
      // A zero or infinite x (infinities are possible with f16 scales, which
      // stay finite) divides to itself; the residual step would lose the
      // sign of a zero (-0 + +0 = +0) and turn an infinity into NaN.
      const bool self = x[e] == 0.f || __builtin_isinf(x[e]);
      y[e] = self ? x[e] : __builtin_fmaf(__builtin_fmaf(-q, scale, x[e]), r, q);
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) y[e] = (scale != 0.f) ? __fdiv_rn(x[e], scale) : 0.f;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) y[e] = fminf(fmaxf(y[e], -kE4m3Max), kE4m3Max);
  uint32_t w[E / 4];
#pragma unroll
  for (int i = 0; i < E / 4; ++i) {
    // Packed conversion: two values per instruction into one 16-bit half.
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * i], y[4 * i + 1], 0, false);
    w[i] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[4 * i + 2], y[4 * i + 3], lo, true);
  }
  if constexpr (E == 4) {
    *(uint32_t*)codes = w[0];
  } else if constexpr (E == 8) {
    *(u32x2*)codes = (u32x2){w[0], w[1]};
  } else {
    *(u32x4*)codes = (u32x4){w[0], w[1], w[2], w[3]};
  }
  if (first) {
    if (f16)
      *(_Float16*)scale_out = (_Float16)scale;
    else
      *(float*)scale_out = scale;
  }
}

// Rows (token, kv head) per wave: each 16-lane quarter of the wave holds one
// row (D/16 values per lane), so a pass covers four rows and a row's absmax
// needs no cross-row exchange. Every load of the wave (the rows' slots, then
// their K and V values) is issued before any of them is waited for.
constexpr int kRowsPerWave = 8;

template <typename QT, bool FP8, int D>
__global__ __launch_bounds__(256) void paged_kv_write_kernel(WriteParams p) {
  constexpr int E = D / 16;                // values per lane
  constexpr int NP = kRowsPerWave / 4;     // passes of four rows
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4;               // row of the pass
  const int li = lane & 15;                // slice of the row: values E*li .. E*li + E - 1
  const int64_t rows = (int64_t)p.N * p.Hkv;
  const int64_t wrow0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * kRowsPerWave;
  // Token and kv head of each row (32-bit: N * Hkv < 2^31 rows is checked on
  // the host).
  int tok[NP], head[NP];
  bool in[NP];
#pragma unroll
  for (int ps = 0; ps < NP; ++ps) {
    const int64_t rr = wrow0 + 4 * ps + grp;
    in[ps] = rr < rows;
    const int row = (int)min(rr, rows - 1);
    tok[ps] = row / p.Hkv;
    head[ps] = row - tok[ps] * p.Hkv;
  }
  int64_t slot[NP];
#pragma unroll
  for (int ps = 0; ps < NP; ++ps) slot[ps] = in[ps] ? p.slots[tok[ps]] : -1;
  // The rows' K and V values, loaded whether or not the slot turns out live
  // (a skipped token's row is read and dropped).
  Raw16<E> wk[NP], wv[NP];
#pragma unroll
  for (int ps = 0; ps < NP; ++ps) {
    if (!in[ps]) continue;
    const int64_t src = (wrow0 + 4 * ps + grp) * D + E * li;
    wk[ps].load((const QT*)p.k + src);
    wv[ps].load((const QT*)p.v + src);
  }
#pragma unroll
  for (int ps = 0; ps < NP; ++ps) {
    const int64_t sl = slot[ps];
    if (!in[ps] || sl < 0 || (p.num_slots != 0 && sl >= p.num_slots)) continue;
    const int h = head[ps];
    // Row of (page, offset, h): (page * bs + offset) * Hkv + h token-major,
    // (page * Hkv + h) * bs + offset head-major.
    const int64_t dst = p.head_major
        ? (((sl >> p.log2bs) * p.Hkv + h) << p.log2bs) + (sl & ((1 << p.log2bs) - 1))
        : sl * p.Hkv + h;
    if constexpr (FP8) {
      const int64_t so = dst * (p.scale_f16 ? 2 : 4);
      float x[E];
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = half_to_f32<QT>(wk[ps].word(e >> 1), e & 1);
      put_fp8_row<E>(x, (uint8_t*)p.k_pages + dst * D + E * li, (char*)p.k_scale + so,
                     p.scale_f16 != 0, li == 0);
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = half_to_f32<QT>(wv[ps].word(e >> 1), e & 1);
      put_fp8_row<E>(x, (uint8_t*)p.v_pages + dst * D + E * li, (char*)p.v_scale + so,
                     p.scale_f16 != 0, li == 0);
    } else {
      wk[ps].store((QT*)p.k_pages + dst * D + E * li);
      wv[ps].store((QT*)p.v_pages + dst * D + E * li);
    }
  }
}

template <typename QT, bool FP8, int D>
hipError_t launch_t(const WriteParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.N * p.Hkv;
  const int64_t grid = (rows + 4 * kRowsPerWave - 1) / (4 * kRowsPerWave);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((paged_kv_write_kernel<QT, FP8, D>), dim3((unsigned)grid), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

template <typename QT>
hipError_t launch_q(const WriteParams& p, bool kv_fp8, int head_dim, hipStream_t stream) {
  switch (head_dim) {
    case 64: return kv_fp8 ? launch_t<QT, true, 64>(p, stream) : launch_t<QT, false, 64>(p, stream);
    case 128: return kv_fp8 ? launch_t<QT, true, 128>(p, stream) : launch_t<QT, false, 128>(p, stream);
    case 256: return kv_fp8 ? launch_t<QT, true, 256>(p, stream) : launch_t<QT, false, 256>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_kv_write(const WriteParams& p, bool q_f16, bool kv_fp8, int head_dim,
                           hipStream_t stream) {
  return q_f16 ? launch_q<_Float16>(p, kv_fp8, head_dim, stream)
               : launch_q<__bf16>(p, kv_fp8, head_dim, stream);
}

}  // namespace pdk
