// Internal interface between the C ABI (paged_decode_abi.cpp) and the
// kernels (decode_kernels.hip). Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace pdk {

// Quotient by a divisor fixed for a launch, as a multiply-high and shift
// (Granlund and Montgomery, "Division by Invariant Integers using
// Multiplication", PLDI 1994): for d >= 2, l = ceil(log2 d) and
// mul = ceil(2^(31 + l) / d), n / d = umulhi(n, mul) >> (l - 1) exactly for
// every 0 <= n < 2^31; d = 1 is marked by shr = -1.
struct FastDiv {
  uint32_t mul;
  int32_t shr;
};

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  const void* ks;    // fp8 scales: f32, or f16 when scale_f16
  const void* vs;
  const int32_t* bt;
  int64_t bt_stride;
  const int32_t* ctx;
  const void* sk;
  const void* sv;
  const int32_t* qlens;   // [B] query tokens per sequence, or null (all Tq)
  const int32_t* slens;   // [B] scratch tokens per sequence, or null (all stok)
  void* out;
  float* lse;
  float* opart;      // O_part [B, Tq, Hq, S, D] when S > 1
  float* lpart;      // LSE_part [B, Tq, Hq, S] when S > 1
  int32_t B, Tq, Hq, Hkv, g, rows, log2bs, S, stok;
  int32_t nrg;       // 16-row groups of the rows = g * Tq packed query rows (an item
                     // carries decode_row_group_factor of them)
  int32_t max_ctx;   // context lengths are clamped to [0, max_ctx] (block-table width * bs)
  int32_t max_page;  // block-table entries are clamped to [0, max_page]
  int32_t causal;    // scratch token j visible to query token t iff j <= t + stok - Tq
  int32_t head_major;  // pages [P, Hkv, bs, D] (else [P, bs, Hkv, D]); scales likewise
  int32_t scale_f16;   // fp8 scales stored as f16 (else f32)
  float scale_log2;  // softmax scale * log2(e)
  // Divisors of the work-item decomposition: Hkv * passes * S (items per
  // rank), passes * Hkv (items per split), passes (row-group passes per kv
  // head) and S.
  FastDiv div_rank, div_split, div_pass, div_s;
};

struct ReduceParams {
  const float* opart;
  const float* lpart;
  void* out;
  float* lse;
  int64_t out_rows;  // B * Tq * Hq output rows
  int32_t S;
};

struct WriteParams {
  const void* k;          // new rows [N, Hkv, D], q dtype
  const void* v;
  const int64_t* slots;   // [N]: page * bs + offset; < 0 skips the token
  void* k_pages;          // [P, bs, Hkv, D], kv dtype
  void* v_pages;
  void* k_scale;          // [P, bs, Hkv], fp8 only: f32, or f16 when scale_f16
  void* v_scale;
  int32_t N, Hkv;
  int32_t log2bs;       // block size = 1 << log2bs
  int32_t head_major;   // pages [P, Hkv, bs, D] (else [P, bs, Hkv, D])
  int32_t scale_f16;    // store the scales as f16
  int64_t num_slots;    // slots >= num_slots are skipped (0: no bound)
};

// Device-side input validation (paged_decode_check). Bits of flags[0].
constexpr uint32_t kCheckContextLens = 1u;   // a context length < 0 or > max_ctx
constexpr uint32_t kCheckBlockTable = 2u;    // a used block-table entry outside the pool
constexpr uint32_t kCheckQLens = 4u;         // a query count outside [0, Tq]
constexpr uint32_t kCheckScratchLens = 8u;   // a scratch count outside [0, stok]

struct CheckParams {
  const int32_t* bt;
  int64_t bt_stride;
  const int32_t* ctx;
  const int32_t* qlens;   // or null
  const int32_t* slens;   // or null
  uint32_t* flags;        // [2]: violated bits, lowest bad sequence
  int32_t B, Tq, stok, log2bs;
  int32_t max_ctx;        // block-table width * bs
  int32_t num_pages;      // pool pages; 0: only negative entries are flagged
};

// The multiplier and shift of FastDiv for divisor d (1 <= d < 2^31).
inline FastDiv make_fast_div(uint32_t d) {
  FastDiv f{0u, -1};
  if (d <= 1) return f;
  int l = 0;
  while ((1ull << l) < d) ++l;
  f.mul = static_cast<uint32_t>(((1ull << (31 + l)) + d - 1) / d);
  f.shr = l - 1;
  return f;
}

hipError_t launch_check(const CheckParams& p, hipStream_t stream);
hipError_t launch_kv_write(const WriteParams& p, bool q_f16, bool kv_fp8, int head_dim,
                           hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, bool q_f16, bool kv_fp8, int head_dim, int grid,
                         hipStream_t stream);
hipError_t launch_reduce(const ReduceParams& p, bool q_f16, int head_dim, int grid,
                         hipStream_t stream);
// Size of the library-owned split workspace of paged_decode_run_noalloc (one
// per device), and the devices it can be set up on.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;
// Device address of that workspace on `device` (looked up once per device,
// with the device current; later calls return the cached address).
hipError_t noalloc_scratch(int device, void** ptr);
// Row groups of 16 packed query rows one work item carries (each K/V tile
// is read once for all of them) for nrg groups at this head dimension and
// page size.
int decode_row_group_factor(int head_dim, int nrg, int log2bs);
// Waves per workgroup of the decode kernel at this head dimension and row
// group factor.
int decode_waves_per_group(int head_dim, int rg);
// Resident workgroups per compute unit of the decode kernel.
int decode_occupancy(bool q_f16, bool kv_fp8, int head_dim, int log2bs, bool scale_f16, int rg);

}  // namespace pdk
