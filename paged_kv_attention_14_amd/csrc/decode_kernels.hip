// Paged-KV split-K decode kernels for gfx950 (MI355X).
//
// The computation is split-K FlashAttention decode: each piece of a
// sequence's context yields a partial output and log-sum-exp, and a combine
// pass merges them ("Implementing a High-Performance Custom Diffusion
// Attention Kernel with FlyDSL", introduction item 3; "Debug Systematically"
// for the LSE intermediate; the decode + reduce kernel pair of "[ROCm] Add
// FlyDSL paged-attention decode backend (dense + fp8) with benchmark",
// Kernels).
//
// Work decomposition. A unit is one (sequence b, kv head hk); split s of S
// covers an equal share of the unit's pages, and the scratch tokens belong to
// the last split. A (unit, split) pair is a work item (with more than 16
// packed query rows, a (unit, split, pass over the row groups) triple). The
// grid is persistent (at most one workgroup per CU, of eight waves at
// D <= 128 with one row group and four otherwise) and each workgroup works
// through its share of the items,
// longest sequence first (see the decode kernel below). The NW waves of a
// workgroup take the tiles of an item round-robin, each with its own
// online-softmax state, and merge in LDS.
//
// Matrix-core mapping (v_mfma_f32_16x16x32_{bf16,f16}, wave64):
//  * The g*Tq query rows that share kv head hk are packed into the 16-wide N
//    side of the tile (head packing, same pull request, Kernels); padding
//    rows repeat the last real row and are never written.
//    More than 16 such rows (the group ratios the pull request's primary
//    kernel cannot head-pack, for which it has a separate cooperative kernel)
//    form 16-row groups. A wave carries two groups at once: every K/V tile is
//    loaded once and multiplied into both, so the pages are read once per
//    pair of groups (four waves per workgroup then, one per SIMD, for the
//    registers of two accumulators). More than two groups take several
//    passes, each a work item, adjacent in the item order.
//  * QK^T is computed operand-swapped: A = K (M = 16 tokens), B = Q (N = rows),
//    as the FlyDSL blog recommends ("Match MFMA Operands to the Desired
//    Fragment Layout"). Lane l then holds scores of row l%16 for tokens
//    4*(l/16)+i, i = 0..3, of each 16-token subtile.
//  * P.V is computed as O^T = V^T P^T with A = V^T (M = 16 head dims) and
//    B = P^T. Its K side is the 32 tokens of the tile. A lane's eight B
//    elements are exactly the eight scores it already holds (subtile 0 then
//    subtile 1), so P never leaves registers; V^T is read from LDS in the
//    matching token order with the gfx950 transposed LDS reads.
//  * The contraction index of both products may be permuted freely as long as
//    both operands use the same permutation, so every operand is loaded in
//    the order that makes its memory access contiguous.
//
// K rows are loaded straight from HBM into the A operand (16 contiguous bytes
// per lane). V rows are loaded with full-row coalescing and staged in a
// per-wave LDS tile. fp8 e4m3fn codes are decoded to the 16-bit MFMA type on
// the way into the operands (exact: every e4m3fn value is representable in
// bf16 and f16); the per-token K scale multiplies the score, the per-token V
// scale multiplies the probability before the cast (the softmax sum uses the
// unscaled probability).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "decode_launch.h"

namespace pdk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

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
constexpr float kLazy = 8.0f;  // base-2 headroom of the lazily moved softmax reference

// Decode 8 e4m3fn codes (two little-endian dwords) to 8 elements of T. The
// gfx950 scaled conversion turns two codes into two packed 16-bit values in
// one instruction; with scale 1 it is exact, as every e4m3fn value is a bf16
// and an f16 value.
template <typename T, bool HI>
__device__ __forceinline__ uint32_t cvt_pair(uint32_t w);
template <>
__device__ __forceinline__ uint32_t cvt_pair<__bf16, false>(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}
template <>
__device__ __forceinline__ uint32_t cvt_pair<__bf16, true>(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}
template <>
__device__ __forceinline__ uint32_t cvt_pair<_Float16, false>(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
}
template <>
__device__ __forceinline__ uint32_t cvt_pair<_Float16, true>(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
}

template <typename T>
__device__ __forceinline__ typename Vec8<T>::type decode8(uint32_t lo, uint32_t hi) {
  const u32x4 r = {cvt_pair<T, false>(lo), cvt_pair<T, true>(lo), cvt_pair<T, false>(hi),
                   cvt_pair<T, true>(hi)};
  return __builtin_bit_cast(typename Vec8<T>::type, r);
}

template <typename T>
__device__ __forceinline__ typename Vec8<T>::type as_vec8(u32x4 x) {
  return __builtin_bit_cast(typename Vec8<T>::type, x);
}

// Raw buffer loads. The descriptor holds a wave-uniform base address (built
// in scalar registers); the per-lane byte offset is a 32-bit VGPR and a
// uniform byte offset rides in the scalar offset field, so a load needs no
// vector address arithmetic. Word 3 is the gfx9 descriptor format for a
// plain byte buffer. The record count is left at its maximum because every
// offset used here is checked by construction, or set to 0 for a load that
// must not happen: a raw buffer load whose offset is not below the record
// count reads no memory and returns zeros. The software pipeline uses that
// to issue the same loads on every path (see the decode kernel).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kAllRecords = 0x7fffffff;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int records = kAllRecords) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, records, kRsrcWord3);
}
__device__ __forceinline__ u32x4 ld_b128(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ float ld_f32(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t ld_b32(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t ld_b16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}

// An fp8 scale as loaded (f32 bits, or f16 bits in the low half) and its value.
// The conversion happens where the scale is used, so a load in flight is not
// waited for early.
template <bool SF16>
__device__ __forceinline__ float scale_value(uint32_t raw) {
  if constexpr (SF16)
    return (float)__builtin_bit_cast(_Float16, (uint16_t)raw);
  else
    return __builtin_bit_cast(float, raw);
}

// Element i of a read-only int32 array at a wave-uniform index, read through
// the constant address space: the load becomes a scalar load, so using the
// value does not wait behind the vector loads the wave has in flight (vector
// loads complete in issue order).
__device__ __forceinline__ int32_t load_uniform(const int32_t* a, int64_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)a)[i];
}

// n / d for 0 <= n < 2^31 through the launch's precomputed reciprocal of d
// (FastDiv): a scalar multiply-high and shift instead of an integer division.
__device__ __forceinline__ int fast_div(int n, uint32_t mul, int shr) {
  const int q = (int)(__umulhi((uint32_t)n, mul) >> (shr < 0 ? 0 : shr));
  return shr < 0 ? n : q;
}

// Value of lane i of each group of four lanes (DPP quad permutation [i,i,i,i]).
__device__ __forceinline__ float quad_bcast(float x, int i) {
  const int v = __builtin_bit_cast(int, x);
  int r;
  switch (i) {
    case 0: r = __builtin_amdgcn_mov_dpp(v, 0x00, 0xf, 0xf, false); break;
    case 1: r = __builtin_amdgcn_mov_dpp(v, 0x55, 0xf, 0xf, false); break;
    case 2: r = __builtin_amdgcn_mov_dpp(v, 0xaa, 0xf, 0xf, false); break;
    default: r = __builtin_amdgcn_mov_dpp(v, 0xff, 0xf, 0xf, false); break;
  }
  return __builtin_bit_cast(float, r);
}

// LDS row of tile token t. fp8 stores row tok(lg, e) (see the P.V operand) at
// 8 * lg + e, so the eight rows one 16-lane group reads are consecutive and
// the 16 rows of a half-wave fall in distinct banks; 16-bit rows keep token
// order, which their two reads per tile already spread over the banks.
template <bool FP8>
__device__ __forceinline__ int lds_row(int t) {
  if constexpr (FP8) return (t < 16) ? (8 * (t >> 2) + (t & 3)) : (8 * ((t - 16) >> 2) + 4 + (t & 3));
  else return t;
}

// Compile-time layout of one kernel instantiation (RG: 16-row query groups
// each wave carries through the tile loop).
template <bool FP8, int D, int NW, int RG = 1>
struct Layout {
  static constexpr int ESZ = FP8 ? 1 : 2;          // bytes per KV element
  static constexpr int ROWB = D * ESZ;             // bytes of one (token, kv head) row
  static constexpr int CPR = ROWB / 16;            // 16-byte chunks per row
  static constexpr int KSTEPS = D / 32;            // MFMA k-steps over the head dim
  static constexpr int DT = D / 16;                // 16-wide head-dim tiles of O
  static constexpr int KL_PER_SUB = FP8 ? KSTEPS / 2 : KSTEPS;  // 16-B K loads per subtile
  static constexpr int KLOADS = 2 * KL_PER_SUB;
  static constexpr int VLOADS = kTile * CPR / 64;
  // LDS row pitch of the staged V tile. The transposed reads fetch 8 bytes per
  // lane from 8 (fp8) or 16 (16-bit) rows at once; these pads put the rows of
  // one read in distinct banks (fp8 additionally stores rows in read order).
  static constexpr int PITCH = ROWB + (FP8 ? 16 : 32);
  static constexpr int STAGE = kTile * PITCH;      // bytes per wave
  static constexpr int MPITCH = D + 4;             // floats per row of the merge buffer
  static constexpr int MERGE = NW * 16 * RG * MPITCH * 4;
  static constexpr int LDSB = (NW * STAGE > MERGE) ? NW * STAGE : MERGE;
  static_assert(VLOADS * 64 == kTile * CPR, "V tile must split evenly over a wave");
};

// Registers of one 32-token tile in flight.
template <bool FP8, int KLOADS, int VLOADS>
struct TileRegs {
  u32x4 k[KLOADS];
  u32x4 v[VLOADS];
  // fp8: K and V scales of half u (tokens 16u .. 16u + 15). Lane (lr, lg)
  // holds token 4*lg + (lr & 3), so the four tokens a lane scores are spread
  // over its quad and reach it by quad broadcasts: one load per half and
  // tensor instead of one per token keeps a tile's memory instructions few.
  uint32_t ks[FP8 ? 2 : 1];   // raw scale bits (see scale_value)
  uint32_t vs[FP8 ? 2 : 1];
};

// Sequences ranked for longest-first dispatch: up to kLptMax sequences are
// ordered by decreasing context length (ties by index); larger batches keep
// their natural order.
constexpr int kLptMax = 1024;

// Waves per workgroup. The decode kernel runs one workgroup per CU: eight
// waves (two per SIMD) while a wave fits in half the register file
// (D <= 128 with one row group), four (one per SIMD) at D = 256 or when a
// wave carries several row groups. One workgroup of eight waves rather than
// two of four: the two workgroups sharing a CU ran their tiles at unequal
// rates (the later-launched one about a quarter slower), so the faster
// finished its items and left the CU half idle at the end.
constexpr int waves_per_group(int D, int RG = 1) { return (D <= 128 && RG == 1) ? 8 : 4; }

// Row groups a wave carries for g*Tq packed rows forming nrg 16-row groups:
// each K/V tile is then read once for both groups of a pair (more groups
// take several passes, each an item of its own). Two groups fit a wave's
// registers without spills at D <= 128 (four spill at D = 128, and two at
// D = 256); D = 256 and pages of fewer than 16 tokens keep one group per item.
constexpr int row_group_factor(int D, int nrg, int log2bs) {
  return (nrg <= 1 || log2bs < 4 || D > 128) ? 1 : 2;
}

// Shared memory of one workgroup.
template <bool FP8, int D, int NW, int RG = 1>
struct Smem {
  __attribute__((aligned(16))) char buf[Layout<FP8, D, NW, RG>::LDSB];  // V stages, then merge
  float ml[2][NW][16 * RG];   // per-wave row max (base 2) and sum
  int lens[kLptMax];     // context length of each sequence
  int order[kLptMax];    // sequence of each rank (decreasing context length)
  int cnt[kLptMax];      // rank of each sequence, while it is counted
};

// One work item: split s of kv-head unit (b, hk). All fields are uniform over
// the workgroup except `my`, which is uniform over a wave.
struct Item {
  int b, hk, s;
  int rg;           // first row group: packed query rows 16*rg .. 16*(rg + RG) - 1
  int lo, hi, end;  // paged tokens [lo, hi), scratch tokens [hi, end)
  int npt, ntiles;  // paged tiles, all tiles
  int my;           // tiles of the calling wave: wave + NW * j for j < my
  bool valid;
};

// Natural-log LSE of merged row r (reads the per-wave max/sum); -inf for a
// row that no wave saw a token of.
template <bool FP8, int D, int NW, int RG>
__device__ __forceinline__ float merged_lse(const Smem<FP8, D, NW, RG>& sm, int r) {
  float M = -__builtin_inff();
  for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.ml[0][w][r]);
  if (M == -__builtin_inff()) return M;
  float Lr = 0.f;
  for (int w = 0; w < NW; ++w) Lr += sm.ml[1][w][r] * fast_exp2(sm.ml[0][w][r] - M);
  return (M + __builtin_amdgcn_logf(Lr)) * kLn2;
}

// Sum the merged rows over waves and hand (row, head-dim offset, 4 values) to
// `put`; hand (row, lse) to `put_lse`.
template <bool FP8, int D, int NW, int RG, typename PutO, typename PutL>
__device__ __forceinline__ void emit_rows(const Smem<FP8, D, NW, RG>& sm, int rows, PutO put,
                                          PutL put_lse) {
  typedef Layout<FP8, D, NW, RG> L;
  const float* mrg = (const float*)sm.buf;
  for (int e = threadIdx.x; e < rows * (D / 4); e += NW * 64) {
    const int r = e / (D / 4);
    const int d4 = (e % (D / 4)) * 4;
    f32x4 o = *(const f32x4*)(mrg + r * L::MPITCH + d4);
#pragma unroll
    for (int w = 1; w < NW; ++w) o += *(const f32x4*)(mrg + (w * 16 * RG + r) * L::MPITCH + d4);
    put(r, d4, o);
  }
  if ((int)threadIdx.x < rows) put_lse((int)threadIdx.x, merged_lse<FP8, D, NW, RG>(sm, threadIdx.x));
}

// Row r of the packed tile <-> output row (query token r / g, q head hk * g + r % g).
__device__ __forceinline__ int64_t out_row_of(int g, int Tq, int Hq, int b, int hk, int r) {
  const int tq = r / g;
  const int h = hk * g + (r % g);
  return ((int64_t)b * Tq + tq) * Hq + h;
}

// ---------------------------------------------------------------------------
// Decode kernel.
//
// Work items are the (unit, split, row group) triples, ranked longest
// sequence first: with R = nrg row groups, item i has rank i / (Hkv*S*R),
// split (i / (Hkv*R)) % S, kv head (i / R) % Hkv and row group i % R, so the
// long splits come first and the short ones fill in behind them
// (longest-processing-time-first). The grid is persistent, at most one
// workgroup per resident slot: workgroup w takes the items of band c (items
// c*G .. c*G + G - 1) in snake order, w on even bands and G - 1 - w on odd
// ones, which evens out the work per workgroup. When every workgroup takes
// at most one item the sequences keep their natural order (no ranking).
//
// Within an item the NW waves take the tiles wave + NW*j, each with its own
// online-softmax state, and merge in LDS at the end of the item. Each wave
// streams its tiles through a two-buffer software pipeline (block-table
// entries two tiles ahead, K/V data one tile ahead) that runs on across item
// boundaries: the last tiles of an item already fetch the query rows, the
// pages and the first tile of the next item, so the merge and the stores of
// one item overlap the first loads of the next.
//
// UPG (pages of at least 16 tokens): a tile starts on a 16-token boundary of
// a page, so each 16-token half of it lies inside one page. Every load
// instruction then reads a single half, whose base address is uniform over
// the wave (kept in scalar registers) while the per-lane part is a fixed
// 32-bit offset; the page of each half is read from the block-table vector
// with a lane read. Smaller pages compute one address per lane and token.
template <typename QT, bool FP8, int D, int NW, bool UPG, bool SF16, int RG>
__global__ __launch_bounds__(NW * 64, 1) void paged_decode_split_kernel(DecodeParams p) {
  static_assert(FP8 || !SF16, "f16 scales belong to an fp8 cache");
  static_assert(sizeof(Smem<FP8, D, NW, RG>) <= 163840, "LDS of one workgroup");
  typedef Layout<FP8, D, NW, RG> L;
  typedef typename Vec8<QT>::type vec8;
  typedef TileRegs<FP8, L::KLOADS, L::VLOADS> Regs;
  constexpr int KSTEPS = L::KSTEPS, DT = L::DT, KL_PER_SUB = L::KL_PER_SUB;
  constexpr int VLOADS = L::VLOADS, CPR = L::CPR, ROWB = L::ROWB, PITCH = L::PITCH;
  constexpr int TPL = 64 / CPR;  // tokens per V load instruction (within one 16-token half)

  __shared__ Smem<FP8, D, NW, RG> sm;

  const int lane = threadIdx.x & 63;
  // Wave index and everything derived from it are uniform over the wave;
  // readfirstlane tells the compiler so (scalar registers, scalar branches).
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15;   // row (N) / token (M) / head dim (M) index within 16
  const int lg = lane >> 4;   // 0..3: which 8-element slice of the K side

  const int B = p.B, S = p.S, Hkv = p.Hkv;
  const int log2bs = p.log2bs;
  const int bsm = (1 << log2bs) - 1;
  const int rows = p.rows;      // packed query rows g*Tq of one kv head
  const int nrg = p.nrg;        // 16-row groups they form
  const char* const kpool = (const char*)p.k;
  const char* const vpool = (const char*)p.v;
  const char* const kscale = (const char*)p.ks;
  const char* const vscale = (const char*)p.vs;
  constexpr int sbytes = SF16 ? 2 : 4;        // bytes per stored scale

  // Rank the sequences: the rank of sequence i is the number of sequences
  // that precede it (longer, or as long and of a lower index). Small batches
  // give each thread one sequence to compare with all others; from 64
  // sequences on, the B*B comparisons are spread over all threads (`parts`
  // threads per sequence, each over a slice of the others, adding their
  // counts in LDS), which costs one more barrier but a shorter loop.
  // The first item's query load needs these arguments; they are read here so
  // their scalar loads overlap the ranking instead of waiting after it.
  struct QArgs {
    int g, Tq, Hq;
    const QT* q;
  };
  QArgs qa0 = {p.g, p.Tq, p.Hq, (const QT*)p.q};

  const int G = gridDim.x;
  const int wg = blockIdx.x;
  const int npass = (nrg + RG - 1) / RG;  // items per (unit, split): RG row groups each
  const int units_s = Hkv * npass * S;
  const int items = B * units_s;

  // With at most one item per workgroup (items <= G) the order does not
  // matter and nothing is ranked.
  const bool ranked = B <= kLptMax && items > G;
  if (ranked) {
    for (int i = threadIdx.x; i < B; i += NW * 64) {
      sm.lens[i] = min(max(p.ctx[i], 0), p.max_ctx);
      sm.cnt[i] = 0;
    }
    __syncthreads();
    const int parts = (B >= 64) ? max(1, NW * 64 / B) : 1;
    for (int x = threadIdx.x; x < B * parts; x += NW * 64) {
      const int i = x % B, part = x / B;
      const int j0 = part * B / parts, j1 = (part + 1) * B / parts;
      const int li = sm.lens[i];
      int before = 0;
#pragma unroll 8
      for (int j = j0; j < j1; ++j) {
        const int lj = sm.lens[j];
        before += (lj > li) || (lj == li && j < i);
      }
      if (parts == 1) sm.order[before] = i;
      else if (before) atomicAdd(&sm.cnt[i], before);
    }
    if (parts > 1) {
      __syncthreads();
      for (int i = threadIdx.x; i < B; i += NW * 64) sm.order[sm.cnt[i]] = i;
    }
    __syncthreads();
  }

  // Query and scratch tokens of sequence b (the handle's Tq and S_tok unless
  // per-sequence counts are given; clamped to them).
  // Kernel arguments read again at a use site, from the kernel argument
  // segment, rather than held in scalar registers through the tile loop,
  // where the larger kernels run short of them (an opaque copy of the
  // segment pointer keeps the reads from being hoisted to the kernel's start).
  typedef __attribute__((address_space(4))) const DecodeParams* KargPtr;
  auto kargs = [&]() -> KargPtr {
    KargPtr pk = (KargPtr)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(pk));
    return pk;
  };

  auto seq_queries = [&](int b) -> int {
    const KargPtr a = kargs();
    return a->qlens ? __builtin_amdgcn_readfirstlane(min(max(load_uniform(a->qlens, b), 0), a->Tq))
                    : a->Tq;
  };
  auto seq_scratch = [&](int b) -> int {
    if constexpr (FP8) return 0;  // an fp8 cache has no scratch tokens
    const KargPtr a = kargs();
    return a->slens
               ? __builtin_amdgcn_readfirstlane(min(max(load_uniform(a->slens, b), 0), a->stok))
               : a->stok;
  };

  auto make_item = [&](int c) -> Item {
    Item it;
    const int i = c * G + ((c & 1) ? G - 1 - wg : wg);
    it.valid = i < items;
    it.b = it.hk = it.s = it.rg = 0;
    it.lo = it.hi = it.end = 0;
    it.npt = it.ntiles = it.my = 0;
    if (!it.valid) return it;
    // Index order (rank, split, kv head, row group): the kv heads of one
    // split, and the row groups of one kv head, are neighbours, so the
    // workgroups that read the same pages (the kv heads' rows of a token are
    // adjacent in token-major pages) do so at about the same time.
    // (The divisors' reciprocals are read from the argument segment here,
    // not held in scalar registers through the tile loop.)
    // (All four reciprocals are read together: one round trip.)
    const KargPtr ka = kargs();
    uint32_t mr = ka->div_rank.mul, ms = ka->div_split.mul, mp = ka->div_pass.mul,
             md = ka->div_s.mul;
    int sr = ka->div_rank.shr, ss = ka->div_split.shr, sp = ka->div_pass.shr, sd = ka->div_s.shr;
    asm volatile("" : "+s"(mr), "+s"(ms), "+s"(mp), "+s"(md), "+s"(sr), "+s"(ss), "+s"(sp),
                 "+s"(sd));
    const int r = fast_div(i, mr, sr);
    const int rem = i - r * units_s;
    it.s = fast_div(rem, ms, ss);
    const int rem2 = rem - it.s * (npass * Hkv);
    it.hk = fast_div(rem2, mp, sp);
    it.rg = (rem2 - it.hk * npass) * RG;
    it.b = ranked ? __builtin_amdgcn_readfirstlane(sm.order[r]) : r;
    const int ctx = ranked ? __builtin_amdgcn_readfirstlane(sm.lens[it.b])
                           : min(max(load_uniform(kargs()->ctx, it.b), 0), kargs()->max_ctx);
    const int npages = (ctx + bsm) >> log2bs;
    const int pps = fast_div(npages + S - 1, md, sd);
    const int p0 = min(it.s * pps, npages);
    const int p1 = min((it.s + 1) * pps, npages);
    it.lo = min(p0 << log2bs, ctx);
    it.hi = min(p1 << log2bs, ctx);
    it.end = it.hi + ((it.s == S - 1) ? seq_scratch(it.b) : 0);
    it.npt = (it.hi - it.lo + kTile - 1) / kTile;
    it.ntiles = it.npt + (it.end - it.hi + kTile - 1) / kTile;
    it.my = (it.ntiles > wave) ? (it.ntiles - wave + NW - 1) / NW : 0;
    return it;
  };

  // Tile j of this wave in item `it`: first token ts (paged tiles: in
  // [lo, hi); scratch tiles: index into the scratch rows) and its number of
  // valid tokens. Returns whether it is a scratch tile.
  auto tile_of = [&](const Item& it, int j, int& ts, int& nvalid) -> bool {
    const int k = wave + NW * j;
    const bool scr = !FP8 && k >= it.npt;
    ts = __builtin_amdgcn_readfirstlane(scr ? (k - it.npt) * kTile : it.lo + k * kTile);
    nvalid = __builtin_amdgcn_readfirstlane(min(kTile, scr ? it.end - it.hi - ts : it.hi - ts));
    return scr;
  };

  // Block-table entries of a paged tile: lane L holds the raw entry of
  // logical page (ts >> log2bs) + min(L, last - first), so lanes past the
  // tile's last page repeat that page; entries are clamped to the pool where
  // they are used (page_of). A scratch tile, or a position with no tile
  // (`live` false), issues the same load with no records and gets zeros.
  // Every lane loads and nothing is selected after the load, so the entry
  // stays in flight until the next pipeline step reads it (a load under a
  // lane condition is waited for at once, and as vector loads complete in
  // order, that wait would also drain the K/V tile fetched ahead).
  auto load_pages = [&](const Item& it, int j, bool live) -> int {
    int ts, nv;
    const bool scr = tile_of(it, j, ts, nv);
    const int first = ts >> log2bs;
    const int last = (ts + nv - 1) >> log2bs;
    const rsrc_t r = make_rsrc(p.bt + (int64_t)it.b * p.bt_stride,
                               (live && !scr) ? kAllRecords : 0);
    return (int)ld_b32(r, (uint32_t)(first + min(lane, last - first)) * 4u, 0);
  };
  auto page_of = [&](int entry) -> int { return min(max(entry, 0), p.max_page); };

  // Query operand of item `it`: lane (row lr, slice lg) holds
  // Q[row][dchunk(step, lg) .. +8], dchunk matching the K loads: dense
  // 32*step + 8*lg; fp8 64*(step/2) + 16*lg + 8*(step%2). Padding rows (past
  // the kv head's g*Tq packed rows) hold a copy of its last row: a row's
  // scores, softmax state and output depend on that row alone, and padding
  // rows are never written, so their values do not matter, and every lane
  // loading a real row keeps the loads unconditional (buffer loads from the
  // sequence's uniform base), in flight until the first product uses them.
  auto qargs = [&]() -> QArgs {
    const KargPtr a = kargs();
    return {a->g, a->Tq, a->Hq, (const QT*)a->q};
  };
  auto load_q = [&](const Item& it, vec8 (*q)[KSTEPS], const QArgs& a) {
    const int g = a.g;
    const rsrc_t qr = make_rsrc(a.q + (int64_t)it.b * a.Tq * a.Hq * D);
#pragma unroll
    for (int gi = 0; gi < RG; ++gi) {
      // packed row: query token pr / g, head pr % g
      const int pr = min(16 * (it.rg + gi) + lr, rows - 1);
      const int tq = pr / g;
      const int h = it.hk * g + (pr % g);
      const uint32_t roff = (uint32_t)((tq * a.Hq + h) * D) * (uint32_t)sizeof(QT);
#pragma unroll
      for (int st = 0; st < KSTEPS; ++st) {
        const int dc = FP8 ? (64 * (st / 2) + 16 * lg + 8 * (st % 2)) : (32 * st + 8 * lg);
        q[gi][st] = as_vec8<QT>(ld_b128(qr, roff + dc * (uint32_t)sizeof(QT), 0));
      }
    }
  };

  // Row of (page, slot, kv head) in the pools and scales: page * bs * Hkv +
  // slot * sstr + hk * hstr, with (sstr, hstr) = (Hkv, 1) token-major and
  // (1, bs) head-major.
  const int sstr = p.head_major ? 1 : Hkv;
  const int hstr = p.head_major ? (1 << log2bs) : 1;
  // Per-lane byte offsets inside a 16-token half (loop invariant).
  const uint32_t tstr = (uint32_t)sstr * ROWB;                     // token stride of a page
  const uint32_t k_off = lr * tstr + 16 * lg;                      // K: token lr, slice lg
  const uint32_t v_off = (lane / CPR) * tstr + (lane % CPR) * 16;  // V: token lane/CPR
  const uint32_t s_off = (4u * lg + (lr & 3)) * sstr * sbytes;     // scales: token 4*lg + lr%4
  const uint32_t xstr = (uint32_t)Hkv * ROWB;                      // token stride of scratch
  const uint32_t xk_off = lr * xstr + 16 * lg;                     // scratch K
  const uint32_t xv_off = (lane / CPR) * xstr + (lane % CPR) * 16;  // scratch V

  // Loads of tile j of item `it` into t. With `live` false (a pipeline
  // position that holds no tile) the buffer loads are issued with no records
  // and return zeros, and scratch tiles issue the same loads as paged ones
  // (only their descriptors and offsets differ), so every path issues the
  // same loads in the same order and the compiler's wait counts stay exact.
  // Pages of fewer than 16 tokens (per-lane addresses) skip the loads of a
  // position that holds no tile instead.
  auto load_tile = [&](const Item& it, int j, int pv, Regs& t, bool live) {
    int ts, nv;
    const bool scr = tile_of(it, j, ts, nv);
    if constexpr (UPG) {
      const bool sc = !FP8 && scr;
      rsrc_t kr[2], vr[2], ksr[2], vsr[2];
      if (sc) {
        // Scratch rows of sequence b, half h = tokens 16h .. 16h + 15 of the
        // tile. The record count ends with the half's last valid row: the
        // rows past it (the next sequence's, or past the buffer) read zeros.
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int nh = min(max(nv - 16 * h, 0), 16);
          const int rec = (live && nh > 0) ? (int)((nh - 1) * xstr + ROWB) : 0;
          const int64_t row0 = ((int64_t)it.b * p.stok + ts + 16 * h) * Hkv + it.hk;
          kr[h] = make_rsrc((const char*)p.sk + row0 * ROWB, rec);
          vr[h] = make_rsrc((const char*)p.sv + row0 * ROWB, rec);
          ksr[h] = vsr[h] = kr[h];  // unused: scratch tiles exist only without fp8
        }
      } else {
        const int nrec = live ? kAllRecords : 0;
        const int first = ts >> log2bs;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int th = ts + 16 * h;
          const int page = page_of(__builtin_amdgcn_readlane(pv, (th >> log2bs) - first));
          const int64_t row = (((int64_t)page << log2bs) * Hkv) + (th & bsm) * sstr + it.hk * hstr;
          kr[h] = make_rsrc(kpool + row * ROWB, nrec);
          vr[h] = make_rsrc(vpool + row * ROWB, nrec);
          if constexpr (FP8) {
            ksr[h] = make_rsrc(kscale + row * sbytes, nrec);
            vsr[h] = make_rsrc(vscale + row * sbytes, nrec);
          }
        }
      }
      // Each load's row offset rides in its per-lane offset, which the
      // record count bounds (the scalar offset only steps within a row).
      const uint32_t ko = sc ? xk_off : k_off;
      const uint32_t vo = sc ? xv_off : v_off;
      const uint32_t rs = sc ? xstr : tstr;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int c = 0; c < KL_PER_SUB; ++c)
          t.k[u * KL_PER_SUB + c] = ld_b128(kr[u], ko, 64 * c);
      }
#pragma unroll
      for (int i = 0; i < VLOADS; ++i)
        t.v[i] = ld_b128(vr[(i * TPL) >> 4], vo + ((i * TPL) & 15) * rs, 0);
      if constexpr (FP8) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          t.ks[u] = SF16 ? ld_b16(ksr[u], s_off, 0) : ld_b32(ksr[u], s_off, 0);
          t.vs[u] = SF16 ? ld_b16(vsr[u], s_off, 0) : ld_b32(vsr[u], s_off, 0);
        }
      }
    } else {
      if (!live) return;
      if (!FP8 && scr) {
        // Scratch rows of sequence b: tokens past the last one are clamped
        // to it, so every read stays inside the scratch buffer.
        const int64_t row0 = ((int64_t)it.b * p.stok + ts) * Hkv + it.hk;
        const rsrc_t kr = make_rsrc((const char*)p.sk + row0 * ROWB);
        const rsrc_t vr = make_rsrc((const char*)p.sv + row0 * ROWB);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const uint32_t o = (uint32_t)min(16 * u + lr, nv - 1) * xstr + 16 * lg;
#pragma unroll
          for (int c = 0; c < KL_PER_SUB; ++c) t.k[u * KL_PER_SUB + c] = ld_b128(kr, o, 64 * c);
        }
#pragma unroll
        for (int i = 0; i < VLOADS; ++i) {
          const uint32_t o = (uint32_t)min(i * TPL + lane / CPR, nv - 1) * xstr + (lane % CPR) * 16;
          t.v[i] = ld_b128(vr, o, 0);
        }
        return;
      }
      // Pages of fewer than 16 tokens: one address per lane and token.
      // Tokens past the tile's end are clamped to its last valid token.
      const int first = ts >> log2bs;
      auto row_of = [&](int idx) -> int64_t {
        const int tok = ts + min(idx, nv - 1);
        const int page = page_of(__shfl(pv, (tok >> log2bs) - first));
        return (((int64_t)page << log2bs) * Hkv) + (tok & bsm) * sstr + it.hk * hstr;
      };
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const char* kr = kpool + row_of(16 * u + lr) * ROWB;
#pragma unroll
        for (int c = 0; c < KL_PER_SUB; ++c)
          t.k[u * KL_PER_SUB + c] = *(const u32x4*)(kr + 64 * c + 16 * lg);
      }
#pragma unroll
      for (int i = 0; i < VLOADS; ++i) {
        const char* vr = vpool + row_of(i * TPL + lane / CPR) * ROWB;
        t.v[i] = *(const u32x4*)(vr + (lane % CPR) * 16);
      }
      if constexpr (FP8) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int64_t r = row_of(16 * u + 4 * lg + (lr & 3));
          t.ks[u] = SF16 ? (uint32_t)((const uint16_t*)kscale)[r] : ((const uint32_t*)kscale)[r];
          t.vs[u] = SF16 ? (uint32_t)((const uint16_t*)vscale)[r] : ((const uint32_t*)vscale)[r];
        }
      }
    }
  };

  // Online-softmax state of this wave for the current item, per row group.
  vec8 qop[RG][KSTEPS];
  f32x4 acc[RG][DT];
  float m_run[RG], l_run[RG];
  char* stage = sm.buf + wave * L::STAGE;

  auto compute_tile = [&](const Item& it, int j, const Regs& t) {
    int ts, nvalid;
    const bool scr = tile_of(it, j, ts, nvalid);
    // Tokens of this tile a row may see: the valid ones, and in a scratch
    // tile under the causal mask only the scratch tokens up to its query
    // token's position. Rows of padding query tokens are computed like the
    // others and replaced by (0, -inf) when the item's rows are written.
    int lim[RG];
#pragma unroll
    for (int gi = 0; gi < RG; ++gi) {
      lim[gi] = nvalid;
      if (!FP8 && scr && p.causal)
        lim[gi] = min(nvalid, (16 * (it.rg + gi) + lr) / p.g + seq_scratch(it.b) -
                                  seq_queries(it.b) + 1 - ts);
    }
    // Stage V rows in LDS (padded pitch). 16-bit rows keep token order; fp8
    // rows are stored in the order the transposed read consumes them. In a
    // tile with fewer than 32 valid tokens the rows past them (another page's
    // data, or anything) are written as zeros: their probability is 0, and a
    // zero row keeps a non-finite value there out of the product.
    if (nvalid == kTile) {
#pragma unroll
      for (int i = 0; i < VLOADS; ++i) {
        const int q = i * 64 + lane;
        *(u32x4*)(stage + lds_row<FP8>(q / CPR) * PITCH + (q % CPR) * 16) = t.v[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < VLOADS; ++i) {
        const int q = i * 64 + lane;
        const u32x4 zero = {0u, 0u, 0u, 0u};
        *(u32x4*)(stage + lds_row<FP8>(q / CPR) * PITCH + (q % CPR) * 16) =
            (q / CPR < nvalid) ? t.v[i] : zero;
      }
    }

    // Scores S[token][row] for the two 16-token subtiles of every row group
    // (each K operand, decoded once, serves all of them).
    f32x4 sc[RG][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int gi = 0; gi < RG; ++gi) sc[gi][u] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < KSTEPS; ++st) {
        vec8 kop;
        if constexpr (FP8) {
          const u32x4 w = t.k[u * KL_PER_SUB + st / 2];
          kop = (st % 2) ? decode8<QT>(w[2], w[3]) : decode8<QT>(w[0], w[1]);
        } else {
          kop = as_vec8<QT>(t.k[u * KL_PER_SUB + st]);
        }
#pragma unroll
        for (int gi = 0; gi < RG; ++gi) sc[gi][u] = mfma16x16x32(kop, qop[gi][st], sc[gi][u]);
      }
    }

    float sv[RG][8];
    float mt[RG];
    bool move = false;
#pragma unroll
    for (int gi = 0; gi < RG; ++gi) {
      mt[gi] = -__builtin_inff();
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tl = 16 * u + 4 * lg + i;
          float x = sc[gi][u][i] * p.scale_log2;
          if constexpr (FP8) x *= quad_bcast(scale_value<SF16>(t.ks[u]), i);
          x = (tl < lim[gi]) ? x : -__builtin_inff();
          sv[gi][u * 4 + i] = x;
          mt[gi] = fmaxf(mt[gi], x);
        }
      }
      mt[gi] = fmaxf(mt[gi], __shfl_xor(mt[gi], 16));
      mt[gi] = fmaxf(mt[gi], __shfl_xor(mt[gi], 32));
      move = move || (mt[gi] > m_run[gi] + kLazy);
    }
    // Online softmax with a lazily moved reference: m_run only moves (and
    // acc, l_run are rescaled by 2^(m_run - m_new)) when some row's tile
    // maximum exceeds it by more than kLazy, so the exponentials stay
    // <= 2^kLazy and most tiles skip the rescale. The first tile always moves
    // it (m_run = -inf). The result is the same quotient; only rounding differs.
    if (__builtin_amdgcn_ballot_w64(move) != 0) {
#pragma unroll
      for (int gi = 0; gi < RG; ++gi) {
        const float m_new = fmaxf(m_run[gi], mt[gi]);
        // A row that has seen no token keeps m = -inf (masked scratch only).
        const float alpha = (m_new == -__builtin_inff()) ? 1.f : fast_exp2(m_run[gi] - m_new);
#pragma unroll
        for (int n = 0; n < DT; ++n) acc[gi][n] *= alpha;
        l_run[gi] *= alpha;
        m_run[gi] = m_new;
      }
    }
    vec8 pop[RG];
#pragma unroll
    for (int gi = 0; gi < RG; ++gi) {
      float lsum = 0.f;
      const float m_ref = (m_run[gi] == -__builtin_inff()) ? 0.f : m_run[gi];  // all -inf: p = 0
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = fast_exp2(sv[gi][e] - m_ref);
        lsum += pe;
        float pw = pe;
        // The V scale of a token past the tile's end may be anything: select.
        if constexpr (FP8)
          pw = (16 * (e >> 2) + 4 * lg + (e & 3) < nvalid)
                   ? pw * quad_bcast(scale_value<SF16>(t.vs[e >> 2]), e & 3) : 0.f;
        pop[gi][e] = (QT)pw;
      }
      l_run[gi] += lsum;
    }

    __builtin_amdgcn_wave_barrier();
    // V^T operand for head-dim tile n: lane (lr, lg) needs V[tok(lg, e)][16n + lr]
    // with tok(lg, e) = 4lg + e (e < 4) or 16 + 4lg + (e - 4) (e >= 4). The
    // gfx950 transposed LDS reads deliver exactly that: within each 16-lane
    // group, lane i receives element (i % 4) of the 8-byte fetches of lanes
    // i/4 + 4e (16-bit), or byte (i % 8) of the fetches of lanes 2e + i/8
    // (8-bit), so each lane addresses the row slice its partners need.
#pragma unroll
    for (int n = 0; n < DT; ++n) {
      vec8 vop;
      if constexpr (FP8) {
        const char* a = stage + (8 * lg + (lr >> 1)) * PITCH + 16 * n + 8 * (lr & 1);
        const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)a);
        vop = decode8<QT>((uint32_t)r[0], (uint32_t)r[1]);
      } else {
        const char* a = stage + (4 * lg + (lr >> 2)) * PITCH + (16 * n + 4 * (lr & 3)) * 2;
        const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a);
        const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + 16 * PITCH));
        const s16x8 both = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
        vop = __builtin_bit_cast(vec8, both);
      }
#pragma unroll
      for (int gi = 0; gi < RG; ++gi) acc[gi][n] = mfma16x16x32(vop, pop[gi], acc[gi][n]);
    }
    __builtin_amdgcn_wave_barrier();
  };

  // Pipeline positions of this wave relative to item `cur`: 0 .. cur.my - 1
  // are its own tiles, cur.my and cur.my + 1 the first two tiles of `nxt`
  // (when this wave has them); anything further is not fetched ahead. Each
  // position selects its item, so the load code exists once.
  auto pos_item = [&](const Item& cur, const Item& nxt, int k, int lim, int& j) -> Item {
    const bool own = k < cur.my;
    j = own ? k : k - cur.my;
    Item it = own ? cur : nxt;
    it.valid = own || j < min(nxt.my, lim);
    return it;
  };
  auto pos_pages = [&](const Item& cur, const Item& nxt, int k) -> int {
    int j;
    const Item it = pos_item(cur, nxt, k, 2, j);
    return load_pages(it, j, it.valid);
  };
  auto pos_tile = [&](const Item& cur, const Item& nxt, int k, int pv, Regs& t) {
    int j;
    const Item it = pos_item(cur, nxt, k, 1, j);
    load_tile(it, j, pv, t, it.valid);
  };

  Regs ta, tb;
  int pv1 = 0;
  bool have0 = false;     // tile 0 of cur already fetched
  bool have1 = false;     // pages of position 1 already fetched (in pv1)
  bool first_in_a = true; // which buffer holds tile 0 of cur

  // Pipeline step at position j of item `cur`: fetch the pages of position
  // j + 2 and the data of position j + 1 (into Y), then compute tile j (in X).
  auto step = [&](const Item& cur, const Item& nxt, int j, const Regs& X, Regs& Y) {
    const int pv2 = pos_pages(cur, nxt, j + 2);
    pos_tile(cur, nxt, j + 1, pv1, Y);
    compute_tile(cur, j, X);
    pv1 = pv2;
  };

  Item cur = make_item(0);
  asm volatile("" : "+s"(qa0.g), "+s"(qa0.Tq), "+s"(qa0.Hq), "+s"(qa0.q));
  if (cur.my > 0) {
    // The block-table entries of the first two tiles go out first; the
    // query rows are fetched while they are in flight, then the first tile
    // itself (the next item's set-up at the top of the loop overlaps its
    // latency). With the second tile's entries issued ahead of the first
    // tile's data, the first pipeline step can issue the second tile without
    // waiting for the first (vector-memory loads complete in issue order).
    const int pv0 = load_pages(cur, 0, true);
    pv1 = load_pages(cur, 1, cur.my > 1);
    load_q(cur, qop, qa0);
    load_tile(cur, 0, pv0, ta, true);
    have0 = true;
    have1 = cur.my > 1;
  }
  for (int c = 0; cur.valid; ++c) {
    const Item nxt = make_item(c + 1);
#pragma unroll
    for (int gi = 0; gi < RG; ++gi) {
#pragma unroll
      for (int n = 0; n < DT; ++n) acc[gi][n] = (f32x4){0.f, 0.f, 0.f, 0.f};
      m_run[gi] = -__builtin_inff();
      l_run[gi] = 0.f;
    }

    // Position 0 (this item's tile 0, or the next item's when this wave has
    // no tiles here) and the pages of position 1, unless fetched already.
    if (!have0) {
      first_in_a = true;
      pos_tile(cur, nxt, 0, pos_pages(cur, nxt, 0), ta);
    }
    if (!have1) pv1 = pos_pages(cur, nxt, 1);
    // Positions alternate between the buffers; the loop runs ta, tb pairs, so
    // an item whose tile 0 sits in tb takes one step first.
    int j = 0;
    if (!first_in_a && cur.my > 0) {
      step(cur, nxt, 0, tb, ta);
      j = 1;
    }
    for (; j < cur.my; j += 2) {
      step(cur, nxt, j, ta, tb);
      if (j + 1 >= cur.my) break;
      step(cur, nxt, j + 1, tb, ta);
    }
    // The query operand is dead until the next item: fetch the next item's
    // rows now, so the load overlaps this item's merge and stores.
    if (nxt.my > 0) load_q(nxt, qop, qargs());
    // Position cur.my (the next item's tile 0) went to the buffer after the
    // last one computed; position cur.my + 1 (its tile 1) has pages in pv1.
    if (cur.my & 1) first_in_a = !first_in_a;
    have0 = nxt.my > 0;
    have1 = nxt.my > 1;

    // The arguments the item's epilogue alone needs (see kargs), all read
    // here: the empty asm takes them as operands, so their scalar loads are
    // issued together and waited for once, overlapping the first merge
    // barrier, instead of one round trip each at its use.
    const KargPtr pa = kargs();
    int eg = pa->g, eTq = pa->Tq, eHq = pa->Hq;
    const int32_t* eql = pa->qlens;
    void* eout = pa->out;
    float* elsep = pa->lse;
    float* eop = pa->opart;
    float* elp = pa->lpart;
    asm volatile("" : "+s"(eg), "+s"(eTq), "+s"(eHq), "+s"(eql), "+s"(eout), "+s"(elsep),
                 "+s"(eop), "+s"(elp));
    // The stores go through global-space pointers: through generic ones they
    // would be flat stores, and while a flat access is outstanding every
    // vector-memory wait the compiler places is a full drain (which would
    // reach into the next item's first tile steps).
    typedef __attribute__((address_space(1))) QT* gQT;
    typedef __attribute__((address_space(1))) float* gf32;
    typedef __attribute__((address_space(1))) f32x4* gf32x4;
    const gQT gout = (gQT)eout;
    const gf32 glse = (gf32)elsep;
    const gf32 gop = (gf32)eop;
    const gf32 glp = (gf32)elp;
    // Row r of the item is packed row r0 + r of its kv head (its RG groups'
    // rows that exist).
    const int r0 = 16 * cur.rg;
    const int nrow = min(16 * RG, rows - r0);
    auto orow = [&](int r) { return out_row_of(eg, eTq, eHq, cur.b, cur.hk, r0 + r); };

    if (cur.ntiles == 0) {
      // Empty split: O_s = 0, LSE_s = -inf (or the final output when S == 1).
      for (int e = threadIdx.x; e < nrow * D; e += NW * 64) {
        const int r = e / D, d = e % D;
        if (S == 1) gout[orow(r) * D + d] = (QT)0.0f;
        else gop[(orow(r) * S + cur.s) * D + d] = 0.0f;
      }
      if ((int)threadIdx.x < nrow) {
        const int64_t o = orow(threadIdx.x);
        if (S == 1) { if (elsep) glse[o] = -__builtin_inff(); }
        else glp[o * S + cur.s] = -__builtin_inff();
      }
    } else {
      // Merge the waves: the four lanes of a row share m_run; sum their l.
#pragma unroll
      for (int gi = 0; gi < RG; ++gi) {
        l_run[gi] += __shfl_xor(l_run[gi], 16);
        l_run[gi] += __shfl_xor(l_run[gi], 32);
        if (lg == 0) {
          sm.ml[0][wave][16 * gi + lr] = m_run[gi];
          sm.ml[1][wave][16 * gi + lr] = l_run[gi];
        }
      }
      __syncthreads();
      // Merge weight of this wave: 2^(m_w - M) / L with M = max m_w and
      // L = sum l_w 2^(m_w - M). A wave that saw no token of the row has
      // m = -inf, weight 0; a row no wave saw (masked scratch only) gets 0.
      float* mrg = (float*)sm.buf;
#pragma unroll
      for (int gi = 0; gi < RG; ++gi) {
        const int rr = 16 * gi + lr;
        float M = -__builtin_inff();
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.ml[0][w][rr]);
        const float Mref = (M == -__builtin_inff()) ? 0.f : M;
        float Lsum = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) Lsum += sm.ml[1][w][rr] * fast_exp2(sm.ml[0][w][rr] - Mref);
        const float wgt = (Lsum > 0.f) ? fast_exp2(m_run[gi] - Mref) / Lsum : 0.f;
#pragma unroll
        for (int n = 0; n < DT; ++n) {
          const f32x4 o = acc[gi][n] * wgt;
          *(f32x4*)(mrg + (wave * 16 * RG + rr) * L::MPITCH + 16 * n + 4 * lg) = o;
        }
      }
      __syncthreads();
      // Rows of padding query tokens (t >= the sequence's count) become (0, -inf).
      const int nq =
          eql ? __builtin_amdgcn_readfirstlane(min(max(load_uniform(eql, cur.b), 0), eTq)) : eTq;
      const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
      if (S == 1) {
        emit_rows<FP8, D, NW, RG>(
            sm, nrow,
            [&](int r, int d4, f32x4 o) {
              if ((r0 + r) / eg >= nq) o = zero4;
              const gQT dst = gout + orow(r) * D + d4;
              dst[0] = (QT)o[0]; dst[1] = (QT)o[1]; dst[2] = (QT)o[2]; dst[3] = (QT)o[3];
            },
            [&](int r, float lse) {
              if (elsep) glse[orow(r)] = ((r0 + r) / eg >= nq) ? -__builtin_inff() : lse;
            });
      } else {
        emit_rows<FP8, D, NW, RG>(
            sm, nrow,
            [&](int r, int d4, f32x4 o) {
              if ((r0 + r) / eg >= nq) o = zero4;
              *(gf32x4)(gop + (orow(r) * S + cur.s) * D + d4) = o;
            },
            [&](int r, float lse) {
              glp[orow(r) * S + cur.s] =
                  ((r0 + r) / eg >= nq) ? -__builtin_inff() : lse;
            });
      }
      __syncthreads();  // the merge buffer is the next item's V stage
    }
    cur = nxt;
  }
}

// ---------------------------------------------------------------------------
// Combine kernel: one wave per output row (b, t, h), four rows per
// workgroup. For the weighted sum of the partial outputs the wave is viewed
// as NG groups of CH = D/4 lanes: lane (group gr, chunk c) owns head dims
// 4c..4c+3 of the splits s = gr, gr + NG, ...; the groups are summed with
// shuffles at the end. The row's log-sum-exps and partial outputs are read
// through buffer descriptors bounded to the row, so a split index past S
// reads as zero without a memory access and every load is unconditional:
// when all S splits fit in one batch of K loads per lane (S <= NG * K, with
// K the smallest of 4, 8, 16 and KB that fits: up to 64 splits at D <= 128,
// 16 at D = 256), every load of the row is issued at once and the maximum, the
// weights and the sum follow from registers, one memory round trip. (The
// zeros past S add nothing, so the result does not depend on K.) Larger S
// reduce the log-sum-exps first, then stream the partial outputs in batches
// of KB.

// One batch of K splits per lane: maximum, weights, weight sum and weighted
// sum of this lane's splits (sums over the NG groups by shuffles, except the
// weighted sum). Returns false when no split has a token (M = -inf).
template <int K, int D>
__device__ __forceinline__ bool combine_splits(rsrc_t lr, rsrc_t orr, int S, int gr, int c,
                                               float& M, float& wsum, f32x4& acc) {
  constexpr int CH = D / 4;
  constexpr int NG = 64 / CH;
  constexpr float kNegInf = -__builtin_inff();
  f32x4 v[K];
  float w[K];
#pragma unroll
  for (int u = 0; u < K; ++u) {
    const int s = gr + u * NG;
    w[u] = ld_f32(lr, (uint32_t)s * 4u, 0);
    v[u] = __builtin_bit_cast(f32x4, ld_b128(orr, (uint32_t)(s * D + 4 * c) * 4u, 0));
  }
  // Every load is issued before the first use (the scheduler would otherwise
  // hold the partial-output loads back behind the maximum).
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < K; ++u)
    if (gr + u * NG >= S) w[u] = kNegInf;
  M = kNegInf;
#pragma unroll
  for (int u = 0; u < K; ++u) M = fmaxf(M, w[u]);
#pragma unroll
  for (int o = CH; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
  // No early exit before the sums: a branch here would let the compiler
  // move the partial-output loads behind it (a second round trip). With
  // M = -inf every weight is 0.
#pragma unroll
  for (int u = 0; u < K; ++u) {
    const float wt = (w[u] == kNegInf) ? 0.f : __expf(w[u] - M);
    wsum += wt;
    acc += wt * v[u];
  }
#pragma unroll
  for (int o = CH; o < 64; o <<= 1) wsum += __shfl_xor(wsum, o);
  return M != kNegInf;
}

template <typename QT, int D>
__global__ __launch_bounds__(256) void paged_decode_reduce_kernel(ReduceParams p) {
  constexpr int CH = D / 4;       // float4 chunks per partial row
  constexpr int NG = 64 / CH;     // split groups per wave
  constexpr int KB = (D >= 256) ? 16 : 64 / NG;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= p.out_rows) return;
  const int lane = threadIdx.x & 63;
  const int S = p.S;
  const int c = lane % CH;
  const int gr = lane / CH;
  QT* out = (QT*)p.out + row * D;
  constexpr float kNegInf = -__builtin_inff();

  float M = kNegInf, wsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  bool any;
  if (S <= NG * KB) {
    const rsrc_t lr = make_rsrc(p.lpart + row * S, S * 4);
    const rsrc_t orr = make_rsrc(p.opart + row * S * D, S * D * 4);
    // The smallest batch that holds S (a wave keeps at most 63 loads in
    // flight, so a batch no deeper than needed also avoids stalling on that).
    if (S <= NG * 4)
      any = combine_splits<4, D>(lr, orr, S, gr, c, M, wsum, acc);
    else if (S <= NG * 8)
      any = combine_splits<8, D>(lr, orr, S, gr, c, M, wsum, acc);
    else if (KB > 16 && S <= NG * 16)
      any = combine_splits<16, D>(lr, orr, S, gr, c, M, wsum, acc);
    else
      any = combine_splits<KB, D>(lr, orr, S, gr, c, M, wsum, acc);
  } else {
    const float* lp = p.lpart + row * S;
    const float* op = p.opart + row * S * D + 4 * c;
    for (int s = lane; s < S; s += 64) M = fmaxf(M, lp[s]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    any = M != kNegInf;
    if (any) {
      for (int s = lane; s < S; s += 64) wsum += __expf(lp[s] - M);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) wsum += __shfl_xor(wsum, o);
      for (int s0 = gr; s0 < S; s0 += NG * KB) {
        f32x4 v[KB];
        float w[KB];
#pragma unroll
        for (int u = 0; u < KB; ++u) {
          const int s = s0 + u * NG;
          const bool ok = s < S;
          w[u] = ok ? lp[s] : kNegInf;
          v[u] = ok ? *(const f32x4*)(op + (int64_t)s * D) : (f32x4){0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < KB; ++u) {
          const float wt = (w[u] == kNegInf) ? 0.f : __expf(w[u] - M);
          acc += wt * v[u];
        }
      }
    }
  }
  if (!any) {
    for (int d = lane; d < D; d += 64) out[d] = (QT)0.0f;
    if (lane == 0 && p.lse) p.lse[row] = kNegInf;
    return;
  }
#pragma unroll
  for (int o = CH; o < 64; o <<= 1) {
    acc[0] += __shfl_xor(acc[0], o);
    acc[1] += __shfl_xor(acc[1], o);
    acc[2] += __shfl_xor(acc[2], o);
    acc[3] += __shfl_xor(acc[3], o);
  }
  if (gr == 0) {
    const float inv = 1.0f / wsum;
    QT* dst = out + 4 * c;
    dst[0] = (QT)(acc[0] * inv); dst[1] = (QT)(acc[1] * inv);
    dst[2] = (QT)(acc[2] * inv); dst[3] = (QT)(acc[3] * inv);
  }
  if (lane == 0 && p.lse) p.lse[row] = M + __logf(wsum);
}

// ---------------------------------------------------------------------------
// Launch table.

template <typename QT, bool FP8, int D, bool SF16, int RG>
static hipError_t launch_rg(const DecodeParams& p, int grid, hipStream_t stream) {
  constexpr int NW = waves_per_group(D, RG);
  if constexpr (RG == 1) {
    if (p.log2bs < 4) {
      hipLaunchKernelGGL((paged_decode_split_kernel<QT, FP8, D, NW, false, SF16, 1>), dim3(grid),
                         dim3(NW * 64), 0, stream, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((paged_decode_split_kernel<QT, FP8, D, NW, true, SF16, RG>), dim3(grid),
                     dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

template <typename QT, bool FP8, int D, bool SF16>
static hipError_t launch_decode_s(const DecodeParams& p, int grid, hipStream_t stream) {
  if constexpr (D <= 128) {
    if (row_group_factor(D, p.nrg, p.log2bs) == 2)
      return launch_rg<QT, FP8, D, SF16, 2>(p, grid, stream);
  }
  return launch_rg<QT, FP8, D, SF16, 1>(p, grid, stream);
}

template <typename QT, bool FP8, int D>
static hipError_t launch_decode_t(const DecodeParams& p, int grid, hipStream_t stream) {
  if constexpr (FP8) {
    if (p.scale_f16) return launch_decode_s<QT, true, D, true>(p, grid, stream);
  }
  return launch_decode_s<QT, FP8, D, false>(p, grid, stream);
}

template <typename QT, bool FP8, int D, bool SF16>
static const void* kernel_fn(bool upg, int rg) {
  if constexpr (D <= 128) {
    if (rg == 2)
      return reinterpret_cast<const void*>(
          &paged_decode_split_kernel<QT, FP8, D, waves_per_group(D, 2), true, SF16, 2>);
  }
  constexpr int NW = waves_per_group(D);
  return upg ? reinterpret_cast<const void*>(&paged_decode_split_kernel<QT, FP8, D, NW, true, SF16, 1>)
             : reinterpret_cast<const void*>(&paged_decode_split_kernel<QT, FP8, D, NW, false, SF16, 1>);
}

template <typename QT, bool FP8, int D>
static int occupancy_t(bool upg, bool sf16, int rg) {
  const void* fn = kernel_fn<QT, FP8, D, false>(upg, rg);
  if constexpr (FP8) {
    if (sf16) fn = kernel_fn<QT, true, D, true>(upg, rg);
  }
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, waves_per_group(D, rg) * 64, 0) !=
      hipSuccess)
    return 0;
  return n;
}

#define PDK_DISPATCH(QT, fp8, D, CALL)                       \
  do {                                                       \
    if (fp8) {                                               \
      switch (D) {                                           \
        case 64: CALL(QT, true, 64);                         \
        case 128: CALL(QT, true, 128);                       \
        case 256: CALL(QT, true, 256);                       \
      }                                                      \
    } else {                                                 \
      switch (D) {                                           \
        case 64: CALL(QT, false, 64);                        \
        case 128: CALL(QT, false, 128);                      \
        case 256: CALL(QT, false, 256);                      \
      }                                                      \
    }                                                        \
  } while (0)

hipError_t launch_decode(const DecodeParams& p, bool q_f16, bool kv_fp8, int head_dim, int grid,
                         hipStream_t stream) {
#define PDK_LAUNCH(QT, F, DD) return launch_decode_t<QT, F, DD>(p, grid, stream)
  if (q_f16) PDK_DISPATCH(_Float16, kv_fp8, head_dim, PDK_LAUNCH);
  else PDK_DISPATCH(__bf16, kv_fp8, head_dim, PDK_LAUNCH);
#undef PDK_LAUNCH
  return hipErrorInvalidValue;
}

int decode_row_group_factor(int head_dim, int nrg, int log2bs) {
  return row_group_factor(head_dim, nrg, log2bs);
}

int decode_waves_per_group(int head_dim, int rg) { return waves_per_group(head_dim, rg); }

int decode_occupancy(bool q_f16, bool kv_fp8, int head_dim, int log2bs, bool scale_f16, int rg) {
#define PDK_OCC(QT, F, DD) return occupancy_t<QT, F, DD>(log2bs >= 4, scale_f16, rg)
  if (q_f16) PDK_DISPATCH(_Float16, kv_fp8, head_dim, PDK_OCC);
  else PDK_DISPATCH(__bf16, kv_fp8, head_dim, PDK_OCC);
#undef PDK_OCC
  return 0;
}

template <typename QT, int D>
static hipError_t launch_reduce_t(const ReduceParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((paged_decode_reduce_kernel<QT, D>), dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_reduce(const ReduceParams& p, bool q_f16, int head_dim, int grid,
                         hipStream_t stream) {
  switch (head_dim) {
    case 64:
      return q_f16 ? launch_reduce_t<_Float16, 64>(p, grid, stream)
                   : launch_reduce_t<__bf16, 64>(p, grid, stream);
    case 128:
      return q_f16 ? launch_reduce_t<_Float16, 128>(p, grid, stream)
                   : launch_reduce_t<__bf16, 128>(p, grid, stream);
    case 256:
      return q_f16 ? launch_reduce_t<_Float16, 256>(p, grid, stream)
                   : launch_reduce_t<__bf16, 256>(p, grid, stream);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Library-owned split workspace of paged_decode_run_noalloc, for callers that
// cannot allocate. Each device holds its own copy of the array until the
// process ends; in host code the name is only a stand-in, so every host use
// goes through the address hipGetSymbolAddress returns for the device.

static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(int device, void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  *ptr = nullptr;
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (cur != device) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) {
      (void)hipGetLastError();  // keep the failure out of the next launch's status
      return e;
    }
    addr[device] = a;
  }
  *ptr = addr[device];
  return hipSuccess;
}

}  // namespace pdk
