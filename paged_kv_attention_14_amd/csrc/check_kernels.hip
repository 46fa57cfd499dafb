// Opt-in validation of the decode call's device-side inputs, gfx950 (MI355X).
//
// The decode kernel clamps what it reads (context lengths to the block-table
// width, block-table entries to the pool when its size is given), so bad
// values never send it outside the buffers; they give wrong attention
// instead. This pass reports them. It checks exactly the values the decode
// kernel would read: every context length, the block-table entries of the
// pages that hold context tokens (logical pages p < ceil(ctx_b / bs) after the
// length is clamped), and the per-sequence query and scratch counts when
// given. Keeping such a debug check behind an opt-in switch that is off by
// default and skipped during graph capture follows the slot check of the
// fused KDA decode pull request (ROCm/aiter #6026, "[FlyDSL] feat(flydsl):
// add fused KDA decode kernels on gfx950", Changes, the contract table's
// environment-variable row): it costs a pass over the block table and a wait
// on the host.
//
// Result: flags[0] = OR of the violated-contract bits, flags[1] = lowest
// sequence index with a violation (0xFFFFFFFF for none). A one-thread kernel
// sets both first, so the result needs no cleared buffer from the caller and
// the pair of launches can sit in a captured graph (no memset node).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_launch.h"

namespace pdk {

namespace {

__global__ __launch_bounds__(64) void check_clear_kernel(uint32_t* flags) {
  if (threadIdx.x == 0) {
    flags[0] = 0u;
    flags[1] = 0xFFFFFFFFu;
  }
}

// One workgroup per sequence at a time (grid-stride over the batch); its
// threads stride over the sequence's used block-table entries.
__global__ __launch_bounds__(256) void check_kernel(CheckParams p) {
  for (int b = blockIdx.x; b < p.B; b += gridDim.x) {
    const int ctx = p.ctx[b];
    uint32_t bad = 0;
    if (ctx < 0 || ctx > p.max_ctx) bad |= kCheckContextLens;
    if (p.qlens) {
      const int t = p.qlens[b];
      if (t < 0 || t > p.Tq) bad |= kCheckQLens;
    }
    if (p.slens) {
      const int s = p.slens[b];
      if (s < 0 || s > p.stok) bad |= kCheckScratchLens;
    }
    const int used = min(max(ctx, 0), p.max_ctx);
    const int npages = (used + (1 << p.log2bs) - 1) >> p.log2bs;
    const int32_t* row = p.bt + (int64_t)b * p.bt_stride;
    for (int i = threadIdx.x; i < npages; i += blockDim.x) {
      const int32_t e = row[i];
      if (e < 0 || (p.num_pages > 0 && e >= p.num_pages)) bad |= kCheckBlockTable;
    }
    // Every thread reaches both barriers: the loop bounds are uniform.
    const int any = __syncthreads_or((int)bad);
    if (any) {
      __shared__ uint32_t mask;
      if (threadIdx.x == 0) mask = 0u;
      __syncthreads();
      if (bad) atomicOr(&mask, bad);
      __syncthreads();
      if (threadIdx.x == 0) {
        atomicOr(&p.flags[0], mask);
        atomicMin(&p.flags[1], (uint32_t)b);
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_check(const CheckParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(check_clear_kernel, dim3(1), dim3(64), 0, stream, p.flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.B <= 0) return e;
  const int grid = p.B < 1024 ? p.B : 1024;
  hipLaunchKernelGGL(check_kernel, dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pdk
