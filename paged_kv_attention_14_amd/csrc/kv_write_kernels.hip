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
// (both correctly rounded single-precision divisions), codes = e4m3fn of
// clamp(y, -448, 448) rounded to nearest even by the gfx950 packed
// conversion; a zero row gets scale 0 and codes 0. With f16 scale storage
// the scale is first rounded to f16 (nearest even, at most the largest
// finite f16) and the rounded value both divides x and is stored; a row whose
// rounded scale is 0 gets codes 0.
//
// Each wave handles a few (token, kv head) rows; each lane holds D/64
// consecutive values of a row.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_launch.h"

namespace pdk {

namespace {

constexpr float kE4m3Max = 448.0f;

template <typename T, int E>
struct RowIO;
template <typename T>
struct RowIO<T, 1> {
  static __device__ __forceinline__ void load(const T* p, float* x) { x[0] = (float)p[0]; }
  static __device__ __forceinline__ void copy(const T* s, T* d) { d[0] = s[0]; }
};
template <typename T>
struct RowIO<T, 2> {
  static __device__ __forceinline__ void load(const T* p, float* x) {
    const uint32_t w = *(const uint32_t*)p;
    const T* e = (const T*)&w;
    x[0] = (float)e[0];
    x[1] = (float)e[1];
  }
  static __device__ __forceinline__ void copy(const T* s, T* d) {
    *(uint32_t*)d = *(const uint32_t*)s;
  }
};
template <typename T>
struct RowIO<T, 4> {
  static __device__ __forceinline__ void load(const T* p, float* x) {
    const uint2 w = *(const uint2*)p;
    const T* e = (const T*)&w;
    x[0] = (float)e[0];
    x[1] = (float)e[1];
    x[2] = (float)e[2];
    x[3] = (float)e[3];
  }
  static __device__ __forceinline__ void copy(const T* s, T* d) {
    *(uint2*)d = *(const uint2*)s;
  }
};

// Wave-wide maximum (every lane gets it): DPP moves inside each 16-lane row
// (quad swaps, then the half-row and row mirrors), shuffles across rows.
template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
  const int o = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false);
  return fmaxf(v, __builtin_bit_cast(float, o));
}
__device__ __forceinline__ float wave_max(float v) {
  v = dpp_max<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v = dpp_max<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v = dpp_max<0x141>(v);  // row_half_mirror
  v = dpp_max<0x140>(v);  // row_mirror
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// Quantise one row (this lane's E values) and store codes and scale.
template <int E>
__device__ __forceinline__ void put_fp8_row(const float* x, uint8_t* codes, void* scale_out,
                                            bool f16, int lane) {
  float am = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) am = fmaxf(am, fabsf(x[e]));
  am = wave_max(am);
  float scale = __fdiv_rn(am, kE4m3Max);
  if (f16) scale = (float)(_Float16)fminf(scale, 65504.0f);
  float y[4] = {0.f, 0.f, 0.f, 0.f};
  if (scale != 0.f) {
#pragma unroll
    for (int e = 0; e < E; ++e)
      y[e] = fminf(fmaxf(__fdiv_rn(x[e], scale), -kE4m3Max), kE4m3Max);
  }
  // Packed conversion: two values per instruction into one 16-bit half.
  const uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  if constexpr (E == 1) {
    codes[0] = (uint8_t)(lo & 0xff);
  } else if constexpr (E == 2) {
    *(uint16_t*)codes = (uint16_t)(lo & 0xffff);
  } else {
    const uint32_t both = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], (int)lo, true);
    *(uint32_t*)codes = both;
  }
  if (lane == 0) {
    if (f16)
      *(_Float16*)scale_out = (_Float16)scale;
    else
      *(float*)scale_out = scale;
  }
}

// Rows (token, kv head) handled by one wave: all their loads are issued
// before any reduction, so the loads and the reductions of the rows overlap.
constexpr int kRowsPerWave = 4;

template <typename QT, bool FP8, int D>
__global__ __launch_bounds__(256) void paged_kv_write_kernel(WriteParams p) {
  constexpr int E = D / 64;  // values per lane
  constexpr int R = kRowsPerWave;
  const int64_t rows = (int64_t)p.N * p.Hkv;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
  const int lane = threadIdx.x & 63;
  int64_t dst[R];
  bool live[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = row0 + r;
    live[r] = false;
    dst[r] = 0;
    if (row < rows) {
      const int64_t i = row / p.Hkv;
      const int64_t slot = p.slots[i];
      live[r] = slot >= 0 && (p.num_slots == 0 || slot < p.num_slots);
      const int64_t h = row - i * p.Hkv;
      // Row of (page, offset, h): (page * bs + offset) * Hkv + h token-major,
      // (page * Hkv + h) * bs + offset head-major.
      dst[r] = p.head_major
          ? (((slot >> p.log2bs) * p.Hkv + h) << p.log2bs) + (slot & ((1 << p.log2bs) - 1))
          : slot * p.Hkv + h;
    }
  }
  if constexpr (FP8) {
    float xk[R][E], xv[R][E];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (!live[r]) continue;
      RowIO<QT, E>::load((const QT*)p.k + (row0 + r) * D + lane * E, xk[r]);
      RowIO<QT, E>::load((const QT*)p.v + (row0 + r) * D + lane * E, xv[r]);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (!live[r]) continue;
      const int64_t so = dst[r] * (p.scale_f16 ? 2 : 4);
      put_fp8_row<E>(xk[r], (uint8_t*)p.k_pages + dst[r] * D + lane * E,
                     (char*)p.k_scale + so, p.scale_f16 != 0, lane);
      put_fp8_row<E>(xv[r], (uint8_t*)p.v_pages + dst[r] * D + lane * E,
                     (char*)p.v_scale + so, p.scale_f16 != 0, lane);
    }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (!live[r]) continue;
      RowIO<QT, E>::copy((const QT*)p.k + (row0 + r) * D + lane * E,
                         (QT*)p.k_pages + dst[r] * D + lane * E);
      RowIO<QT, E>::copy((const QT*)p.v + (row0 + r) * D + lane * E,
                         (QT*)p.v_pages + dst[r] * D + lane * E);
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
