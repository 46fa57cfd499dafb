// C ABI of the paged-KV decode library: argument checks, split choice and
// launches. Every host-visible fault is reported before any launch; nothing
// here allocates device memory or synchronises, so run + reduce can be
// captured in a HIP graph. The operation and layouts are documented in
// include/paged_decode.h.

#include "paged_decode.h"

#include <hip/hip_runtime_api.h>

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>

#include "decode_launch.h"

struct pd_handle {
  pd_config cfg;
  int device;
  int num_cus;
  int log2bs;
  int rgf;     // row groups per work item (each K/V tile read once for all of them)
  int slots;   // resident decode workgroups: occupancy x compute units
  void* noalloc_ws;             // device address of this device's library-owned workspace
  hipError_t noalloc_ws_status; // result of looking it up at create
};

namespace {

thread_local char g_err[512] = "";

pd_status fail(pd_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

pd_status ok() {
  g_err[0] = '\0';
  return PD_OK;
}

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kTileTokens = 32;
constexpr int kMaxRowGroups = 8;  // packed query rows per kv head: at most 8 * 16

// 16-row groups of the g * Tq packed query rows of one kv head.
int row_groups(const pd_config& c) {
  return ((c.num_q_heads / c.num_kv_heads) * c.q_tokens + 15) / 16;
}

// Work items per (sequence, kv head, split): the row groups in passes of
// h->rgf groups each.
int row_passes(const pd_handle* h) { return (row_groups(h->cfg) + h->rgf - 1) / h->rgf; }

// Split count for num_splits = 0. A pure function of the handle and batch
// (it never reads context_lens, so it is safe under graph capture): about two
// work items per resident workgroup, so the longest-first dispatch order has
// a second round to even out the length mix; up to four when the items stay
// long (at least 16 tiles per wave at the longest context the handle
// allows), where a split's fixed cost is small against its length; never
// fewer than two 32-token tiles per wave. (Measured best on MI355X at every
// workload shape here.)
int auto_splits(const pd_handle* h, int batch) {
  const pd_config& c = h->cfg;
  const long units = static_cast<long>(batch) * c.num_kv_heads * row_passes(h);
  if (units <= 0) return 1;
  const long waves = pdk::decode_waves_per_group(c.head_dim, h->rgf);
  const long max_tokens =
      static_cast<long>(c.max_blocks_per_seq) * c.block_size + c.scratch_tokens;
  const long max_tiles = (max_tokens + kTileTokens - 1) / kTileTokens;
  const long two = (2L * h->slots + units - 1) / units;
  const long four = (4L * h->slots + units - 1) / units;
  const long long_items = max_tiles / (waves * 16);
  long s = four < long_items ? four : long_items;
  if (s < two) s = two;
  const long cap = max_tiles / (waves * 2);  // two tiles per wave
  if (s > cap) s = cap;
  if (s > c.max_num_splits) s = c.max_num_splits;
  if (s < 1) s = 1;
  return static_cast<int>(s);
}

pd_status resolve_splits(const pd_handle* h, int batch, int requested, int* out) {
  if (requested < 0) return fail(PD_ERR_INVALID_ARG, "num_splits must be >= 0 (got %d)", requested);
  if (requested > h->cfg.max_num_splits)
    return fail(PD_ERR_INVALID_ARG, "num_splits %d exceeds the handle's max_num_splits %d",
                requested, h->cfg.max_num_splits);
  *out = requested ? requested : auto_splits(h, batch);
  return PD_OK;
}

size_t round256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Workspace layout for S > 1: O_part f32 [B, Tq, Hq, S, D] at offset 0, then
// LSE_part f32 [B, Tq, Hq, S] at the next 256-byte boundary. S = 1 needs none.
struct WsLayout {
  size_t o_off, l_off, total;
};

WsLayout workspace_layout(const pd_handle* h, int batch, int splits) {
  const pd_config& c = h->cfg;
  WsLayout w{0, 0, 0};
  if (splits <= 1 || batch <= 0) return w;
  const size_t rows = static_cast<size_t>(batch) * c.q_tokens * c.num_q_heads * splits;
  w.l_off = round256(rows * c.head_dim * sizeof(float));
  w.total = round256(w.l_off + rows * sizeof(float));
  return w;
}

size_t workspace_bytes(const pd_handle* h, int batch, int splits) {
  return workspace_layout(h, batch, splits).total;
}

pd_status check_args(const pd_handle* h, const pd_args* a) {
  if (!h) return fail(PD_ERR_INVALID_ARG, "handle is NULL");
  if (!a) return fail(PD_ERR_INVALID_ARG, "args is NULL");
  const pd_config& c = h->cfg;
  if (a->batch < 0 || a->batch > c.max_batch)
    return fail(PD_ERR_INVALID_ARG, "batch %d outside [0, max_batch=%d]", a->batch, c.max_batch);
  if (a->num_pages < 0) return fail(PD_ERR_INVALID_ARG, "num_pages %d < 0", a->num_pages);
  if (a->batch == 0) return PD_OK;
  if (!a->q || !a->k_pages || !a->v_pages || !a->block_table || !a->context_lens || !a->out)
    return fail(PD_ERR_INVALID_ARG,
                "q, k_pages, v_pages, block_table, context_lens and out are required");
  if (!aligned16(a->q) || !aligned16(a->k_pages) || !aligned16(a->v_pages) ||
      !aligned16(a->out))
    return fail(PD_ERR_INVALID_ARG, "q, k_pages, v_pages and out must be 16-byte aligned");
  if (a->block_table_stride < c.max_blocks_per_seq)
    return fail(PD_ERR_INVALID_ARG, "block_table_stride %lld < max_blocks_per_seq %d",
                static_cast<long long>(a->block_table_stride), c.max_blocks_per_seq);
  const bool fp8 = c.kv_dtype == PD_DTYPE_FP8_E4M3FN;
  if (fp8 && (!a->k_scale || !a->v_scale))
    return fail(PD_ERR_INVALID_ARG, "fp8 KV needs k_scale and v_scale");
  if (!fp8 && (a->k_scale || a->v_scale))
    return fail(PD_ERR_INVALID_ARG, "k_scale/v_scale are for fp8 KV only");
  if (c.scratch_tokens > 0) {
    if (!a->scratch_k || !a->scratch_v)
      return fail(PD_ERR_INVALID_ARG, "scratch_tokens > 0 needs scratch_k and scratch_v");
    if (!aligned16(a->scratch_k) || !aligned16(a->scratch_v))
      return fail(PD_ERR_INVALID_ARG, "scratch_k/scratch_v must be 16-byte aligned");
  } else if (a->scratch_k || a->scratch_v) {
    return fail(PD_ERR_INVALID_ARG, "scratch_k/scratch_v given but scratch_tokens is 0");
  }
  if (!std::isfinite(a->softmax_scale))
    return fail(PD_ERR_INVALID_ARG, "softmax_scale must be finite");
  return PD_OK;
}

pdk::DecodeParams make_params(const pd_handle* h, const pd_args* a, int splits, void* ws) {
  const pd_config& c = h->cfg;
  pdk::DecodeParams p{};
  p.q = a->q;
  p.k = a->k_pages;
  p.v = a->v_pages;
  p.ks = a->k_scale;
  p.vs = a->v_scale;
  p.bt = a->block_table;
  p.bt_stride = a->block_table_stride;
  p.ctx = a->context_lens;
  p.sk = a->scratch_k;
  p.sv = a->scratch_v;
  p.qlens = a->q_lens;
  p.slens = c.scratch_tokens > 0 ? a->scratch_lens : nullptr;
  p.max_page = a->num_pages > 0 ? a->num_pages - 1 : 0x7fffffff;
  p.out = a->out;
  p.lse = a->lse;
  const WsLayout w = workspace_layout(h, a->batch, splits);
  const bool uses_ws = w.total > 0;
  char* base = static_cast<char*>(ws);
  p.opart = uses_ws ? reinterpret_cast<float*>(base + w.o_off) : nullptr;
  p.lpart = uses_ws ? reinterpret_cast<float*>(base + w.l_off) : nullptr;
  p.B = a->batch;
  p.Tq = c.q_tokens;
  p.Hq = c.num_q_heads;
  p.Hkv = c.num_kv_heads;
  p.g = c.num_q_heads / c.num_kv_heads;
  p.rows = p.g * c.q_tokens;
  p.nrg = row_groups(c);
  const long long max_ctx = static_cast<long long>(c.max_blocks_per_seq) * c.block_size;
  p.max_ctx = max_ctx < 0x7fffffffLL ? static_cast<int32_t>(max_ctx) : 0x7fffffff;
  p.log2bs = h->log2bs;
  p.S = splits;
  p.stok = c.scratch_tokens;
  p.causal = c.scratch_mask == PD_SCRATCH_MASK_CAUSAL ? 1 : 0;
  p.head_major = c.kv_layout == PD_KV_LAYOUT_HEAD_MAJOR ? 1 : 0;
  p.scale_f16 = c.scale_dtype == PD_SCALE_F16 ? 1 : 0;
  p.scale_log2 = a->softmax_scale * 1.4426950408889634f;
  const uint32_t passes = static_cast<uint32_t>(row_passes(h));
  p.div_rank = pdk::make_fast_div(static_cast<uint32_t>(c.num_kv_heads) * passes * splits);
  p.div_split = pdk::make_fast_div(passes * c.num_kv_heads);
  p.div_pass = pdk::make_fast_div(passes);
  p.div_s = pdk::make_fast_div(static_cast<uint32_t>(splits));
  return p;
}

pd_status check_workspace(const pd_handle* h, int batch, int splits, const void* workspace,
                          size_t ws_bytes) {
  const size_t need = workspace_bytes(h, batch, splits);
  if (need == 0) return PD_OK;
  if (!workspace || ws_bytes < need)
    return fail(PD_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes needed (num_splits %d), got %zu",
                need, splits, workspace ? ws_bytes : static_cast<size_t>(0));
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(PD_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return PD_OK;
}

// Decode launch over the persistent grid: one workgroup per resident slot at
// most; each takes its share of the B * Hkv * row groups * S work items.
pd_status launch_split_pass(const pd_handle* h, const pd_args* a, int splits, void* workspace,
                            hipStream_t stream) {
  const pd_config& c = h->cfg;
  pdk::DecodeParams p = make_params(h, a, splits, workspace);
  const long long items =
      static_cast<long long>(a->batch) * c.num_kv_heads * row_passes(h) * splits;
  if (items > 0x7fffffffLL) return fail(PD_ERR_UNSUPPORTED, "%lld work items too many", items);
  const long long grid = items < h->slots ? items : h->slots;
  hipError_t e = pdk::launch_decode(p, c.q_dtype == PD_DTYPE_F16,
                                    c.kv_dtype == PD_DTYPE_FP8_E4M3FN, c.head_dim,
                                    static_cast<int>(grid), stream);
  if (e != hipSuccess) return fail(PD_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
  return ok();
}

// Split-K combine launch (S > 1): one wave per output row, four per workgroup.
pd_status launch_combine(const pd_handle* h, const pd_args* a, int splits, const void* workspace,
                         hipStream_t stream) {
  const pd_config& c = h->cfg;
  const WsLayout w = workspace_layout(h, a->batch, splits);
  pdk::ReduceParams r{};
  r.opart = reinterpret_cast<const float*>(static_cast<const char*>(workspace) + w.o_off);
  r.lpart = reinterpret_cast<const float*>(static_cast<const char*>(workspace) + w.l_off);
  r.out = a->out;
  r.lse = a->lse;
  r.out_rows = static_cast<int64_t>(a->batch) * c.q_tokens * c.num_q_heads;
  r.S = splits;
  const long long grid = (r.out_rows + 3) / 4;
  hipError_t e = pdk::launch_reduce(r, c.q_dtype == PD_DTYPE_F16, c.head_dim,
                                    static_cast<int>(grid), stream);
  if (e != hipSuccess) return fail(PD_ERR_HIP, "reduce launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

pd_status paged_decode_create(const pd_config* cfg, pd_handle** out) {
  if (!cfg || !out) return fail(PD_ERR_INVALID_ARG, "cfg and out must not be NULL");
  *out = nullptr;
  const pd_config& c = *cfg;
  if (c.num_q_heads <= 0 || c.num_kv_heads <= 0 || c.num_q_heads % c.num_kv_heads != 0)
    return fail(PD_ERR_INVALID_ARG, "num_kv_heads (%d) must divide num_q_heads (%d)",
                c.num_kv_heads, c.num_q_heads);
  if (c.head_dim != 64 && c.head_dim != 128 && c.head_dim != 256)
    return fail(PD_ERR_UNSUPPORTED, "head_dim %d not in {64, 128, 256}", c.head_dim);
  if (!is_pow2(c.block_size) || c.block_size > 256)
    return fail(PD_ERR_UNSUPPORTED, "block_size %d is not a power of two in [1, 256]",
                c.block_size);
  if (c.q_tokens <= 0)
    return fail(PD_ERR_INVALID_ARG, "q_tokens must be >= 1 (got %d)", c.q_tokens);
  const int rows = (c.num_q_heads / c.num_kv_heads) * c.q_tokens;
  if (rows > 16 * kMaxRowGroups)
    return fail(PD_ERR_UNSUPPORTED, "packed rows (Hq/Hkv)*q_tokens = %d exceed %d", rows,
                16 * kMaxRowGroups);
  if (c.scratch_tokens < 0 || c.scratch_tokens > 64)
    return fail(PD_ERR_UNSUPPORTED, "scratch_tokens %d outside [0, 64]", c.scratch_tokens);
  if (c.q_dtype != PD_DTYPE_BF16 && c.q_dtype != PD_DTYPE_F16)
    return fail(PD_ERR_UNSUPPORTED, "q_dtype must be bf16 or f16");
  if (c.kv_dtype != c.q_dtype && c.kv_dtype != PD_DTYPE_FP8_E4M3FN)
    return fail(PD_ERR_UNSUPPORTED, "kv_dtype must equal q_dtype or be fp8 e4m3fn");
  if (c.kv_dtype == PD_DTYPE_FP8_E4M3FN && c.scratch_tokens > 0)
    return fail(PD_ERR_UNSUPPORTED, "scratch tokens are supported with dense KV only");
  if (c.scratch_mask != PD_SCRATCH_MASK_NONE && c.scratch_mask != PD_SCRATCH_MASK_CAUSAL)
    return fail(PD_ERR_INVALID_ARG, "scratch_mask %d is not a pd_scratch_mask", c.scratch_mask);
  if (c.kv_layout != PD_KV_LAYOUT_TOKEN_MAJOR && c.kv_layout != PD_KV_LAYOUT_HEAD_MAJOR)
    return fail(PD_ERR_INVALID_ARG, "kv_layout %d is not a pd_kv_layout", c.kv_layout);
  if (c.scale_dtype != PD_SCALE_F32 && c.scale_dtype != PD_SCALE_F16)
    return fail(PD_ERR_INVALID_ARG, "scale_dtype %d is not a pd_scale_dtype", c.scale_dtype);
  if (c.scale_dtype == PD_SCALE_F16 && c.kv_dtype != PD_DTYPE_FP8_E4M3FN)
    return fail(PD_ERR_INVALID_ARG, "f16 scales are for an fp8 cache only");
  if (c.max_batch <= 0 || c.max_blocks_per_seq <= 0)
    return fail(PD_ERR_INVALID_ARG, "max_batch and max_blocks_per_seq must be positive");
  if (c.max_num_splits < 1 || c.max_num_splits > 256)
    return fail(PD_ERR_INVALID_ARG, "max_num_splits %d outside [1, 256]", c.max_num_splits);
  if (static_cast<long long>(c.max_blocks_per_seq) * c.block_size + c.scratch_tokens >
      0x7fffffffLL)
    return fail(PD_ERR_UNSUPPORTED, "context capacity exceeds 2^31 tokens");

  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(PD_ERR_UNSUPPORTED, "no HIP device: %s", hipGetErrorString(e));
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess)
    return fail(PD_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(PD_ERR_UNSUPPORTED, "device %d is %s; this library runs on gfx950 only", dev,
                prop.gcnArchName);

  pd_handle* h = new (std::nothrow) pd_handle;
  if (!h) return fail(PD_ERR_INVALID_ARG, "out of host memory");
  h->cfg = c;
  h->device = dev;
  h->num_cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
  h->log2bs = ilog2(c.block_size);
  h->rgf = pdk::decode_row_group_factor(c.head_dim, row_groups(c), h->log2bs);
  const int occ = pdk::decode_occupancy(c.q_dtype == PD_DTYPE_F16,
                                        c.kv_dtype == PD_DTYPE_FP8_E4M3FN, c.head_dim,
                                        h->log2bs, c.scale_dtype == PD_SCALE_F16, h->rgf);
  if (occ <= 0) {
    delete h;
    return fail(PD_ERR_HIP, "occupancy query for the decode kernel failed");
  }
  h->slots = occ * h->num_cus;
  // The device's copy of the library-owned workspace (paged_decode_run_noalloc),
  // looked up once per device with the device current. A failure here only
  // disables that entry point.
  h->noalloc_ws = nullptr;
  h->noalloc_ws_status = pdk::noalloc_scratch(dev, &h->noalloc_ws);
  *out = h;
  return ok();
}

void paged_decode_destroy(pd_handle* h) { delete h; }

pd_status paged_decode_num_splits(const pd_handle* h, int32_t batch, int32_t requested,
                                  int32_t* resolved) {
  if (!h || !resolved) return fail(PD_ERR_INVALID_ARG, "handle and resolved must not be NULL");
  if (batch < 0 || batch > h->cfg.max_batch)
    return fail(PD_ERR_INVALID_ARG, "batch %d outside [0, max_batch=%d]", batch,
                h->cfg.max_batch);
  int s = 0;
  pd_status st = resolve_splits(h, batch, requested, &s);
  if (st != PD_OK) return st;
  *resolved = s;
  return ok();
}

pd_status paged_decode_workspace_size(const pd_handle* h, int32_t batch, int32_t num_splits,
                                      size_t* bytes) {
  if (!h || !bytes) return fail(PD_ERR_INVALID_ARG, "handle and bytes must not be NULL");
  if (batch < 0 || batch > h->cfg.max_batch)
    return fail(PD_ERR_INVALID_ARG, "batch %d outside [0, max_batch=%d]", batch,
                h->cfg.max_batch);
  int s = 0;
  pd_status st = resolve_splits(h, batch, num_splits, &s);
  if (st != PD_OK) return st;
  *bytes = batch > 0 ? workspace_bytes(h, batch, s) : 0;
  return ok();
}

pd_status paged_decode_run(pd_handle* h, const pd_args* a, void* workspace,
                           size_t ws_bytes, hipStream_t stream) {
  pd_status st = check_args(h, a);
  if (st != PD_OK) return st;
  if (a->batch == 0) return ok();
  int s = 0;
  st = resolve_splits(h, a->batch, a->num_splits, &s);
  if (st != PD_OK) return st;
  st = check_workspace(h, a->batch, s, workspace, ws_bytes);
  if (st != PD_OK) return st;
  return launch_split_pass(h, a, s, workspace, stream);
}

pd_status paged_decode_reduce(pd_handle* h, const pd_args* a, void* workspace,
                              size_t ws_bytes, hipStream_t stream) {
  pd_status st = check_args(h, a);
  if (st != PD_OK) return st;
  if (a->batch == 0) return ok();
  int s = 0;
  st = resolve_splits(h, a->batch, a->num_splits, &s);
  if (st != PD_OK) return st;
  if (s == 1) return ok();
  st = check_workspace(h, a->batch, s, workspace, ws_bytes);
  if (st != PD_OK) return st;
  return launch_combine(h, a, s, workspace, stream);
}

pd_status paged_decode_run_noalloc(pd_handle* h, const pd_args* a, hipStream_t stream) {
  pd_status st = check_args(h, a);
  if (st != PD_OK) return st;
  if (a->batch == 0) return ok();
  int s = 0;
  st = resolve_splits(h, a->batch, a->num_splits, &s);
  if (st != PD_OK) return st;
  const size_t need = workspace_bytes(h, a->batch, s);
  if (need > pdk::kNoAllocScratchBytes)
    return fail(PD_ERR_WORKSPACE_TOO_SMALL,
                "paged_decode_run_noalloc: %zu bytes of split workspace needed (batch %d, "
                "num_splits %d), above its fixed maximum of %zu; use fewer splits or a "
                "smaller batch, or paged_decode_run with a caller workspace",
                need, a->batch, s, pdk::kNoAllocScratchBytes);
  if (need > 0) {
    if (h->noalloc_ws_status != hipSuccess || !h->noalloc_ws)
      return fail(PD_ERR_HIP, "paged_decode_run_noalloc: no workspace address on device %d: %s",
                  h->device, hipGetErrorString(h->noalloc_ws_status));
    int cur = -1;
    const hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess || cur != h->device)
      return fail(PD_ERR_INVALID_ARG,
                  "paged_decode_run_noalloc: the current device (%d) is not the handle's (%d)",
                  cur, h->device);
  }
  st = launch_split_pass(h, a, s, h->noalloc_ws, stream);
  if (st != PD_OK || s == 1) return st;
  return launch_combine(h, a, s, h->noalloc_ws, stream);
}

pd_status paged_decode_write_kv(pd_handle* h, const pd_write_args* a, hipStream_t stream) {
  if (!h || !a) return fail(PD_ERR_INVALID_ARG, "handle and args must not be NULL");
  const pd_config& c = h->cfg;
  if (a->num_tokens < 0) return fail(PD_ERR_INVALID_ARG, "num_tokens %d < 0", a->num_tokens);
  if (a->num_slots < 0)
    return fail(PD_ERR_INVALID_ARG, "num_slots %lld < 0", static_cast<long long>(a->num_slots));
  if (a->num_tokens == 0) return ok();
  if (static_cast<long long>(a->num_tokens) * c.num_kv_heads > INT_MAX)
    return fail(PD_ERR_INVALID_ARG, "num_tokens * num_kv_heads = %lld rows exceeds 2^31 - 1",
                static_cast<long long>(a->num_tokens) * c.num_kv_heads);
  if (!a->k || !a->v || !a->slot_mapping || !a->k_pages || !a->v_pages)
    return fail(PD_ERR_INVALID_ARG, "k, v, slot_mapping, k_pages and v_pages are required");
  if ((reinterpret_cast<uintptr_t>(a->k) | reinterpret_cast<uintptr_t>(a->v) |
       reinterpret_cast<uintptr_t>(a->k_pages) | reinterpret_cast<uintptr_t>(a->v_pages)) & 15u)
    return fail(PD_ERR_INVALID_ARG, "k, v, k_pages and v_pages must be 16-byte aligned");
  const bool fp8 = c.kv_dtype == PD_DTYPE_FP8_E4M3FN;
  if (fp8 && (!a->k_scale || !a->v_scale))
    return fail(PD_ERR_INVALID_ARG, "an fp8 cache needs k_scale and v_scale");
  if (!fp8 && (a->k_scale || a->v_scale))
    return fail(PD_ERR_INVALID_ARG, "k_scale/v_scale given for a dense cache");
  pdk::WriteParams p{};
  p.k = a->k;
  p.v = a->v;
  p.slots = a->slot_mapping;
  p.k_pages = a->k_pages;
  p.v_pages = a->v_pages;
  p.k_scale = a->k_scale;
  p.v_scale = a->v_scale;
  p.N = a->num_tokens;
  p.Hkv = c.num_kv_heads;
  p.log2bs = h->log2bs;
  p.head_major = c.kv_layout == PD_KV_LAYOUT_HEAD_MAJOR ? 1 : 0;
  p.scale_f16 = c.scale_dtype == PD_SCALE_F16 ? 1 : 0;
  p.num_slots = a->num_slots;
  hipError_t e = pdk::launch_kv_write(p, c.q_dtype == PD_DTYPE_F16, fp8, c.head_dim, stream);
  if (e != hipSuccess) return fail(PD_ERR_HIP, "kv write launch failed: %s", hipGetErrorString(e));
  return ok();
}

pd_status paged_decode_check(pd_handle* h, const pd_args* a, uint32_t* flags,
                             hipStream_t stream) {
  pd_status st = check_args(h, a);
  if (st != PD_OK) return st;
  if (!flags) return fail(PD_ERR_INVALID_ARG, "flags is NULL");
  if ((reinterpret_cast<uintptr_t>(flags) & 3u) != 0)
    return fail(PD_ERR_INVALID_ARG, "flags must be 4-byte aligned");
  const pd_config& c = h->cfg;
  pdk::CheckParams p{};
  p.bt = a->block_table;
  p.bt_stride = a->block_table_stride;
  p.ctx = a->context_lens;
  p.qlens = a->q_lens;
  p.slens = a->scratch_lens;
  p.flags = flags;
  p.B = a->batch;
  p.Tq = c.q_tokens;
  p.stok = c.scratch_tokens;
  p.log2bs = h->log2bs;
  const long long max_ctx = static_cast<long long>(c.max_blocks_per_seq) * c.block_size;
  p.max_ctx = max_ctx < 0x7fffffffLL ? static_cast<int32_t>(max_ctx) : 0x7fffffff;
  p.num_pages = a->num_pages;
  hipError_t e = pdk::launch_check(p, stream);
  if (e != hipSuccess) return fail(PD_ERR_HIP, "check launch failed: %s", hipGetErrorString(e));
  return ok();
}

const char* paged_decode_last_error(void) { return g_err; }

}  // extern "C"
