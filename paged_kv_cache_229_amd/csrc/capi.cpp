// C-ABI entry points: host-side argument checks, workspace layout and kernel launches.
//
// Every check runs on the host before the first HIP call, so an invalid call never enqueues anything and
// can be exercised without a GPU.  Nothing here reads device memory or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <string>

#include "kernels.h"
#include "paged_kv.h"

namespace {

constexpr int kAbiVersion = 6;

thread_local std::string g_error;
thread_local int g_partition_keys = 0;
thread_local int g_target_items = 0;
thread_local int g_tile_kind = 0;
thread_local hipEvent_t g_ev_start = nullptr;
thread_local hipEvent_t g_ev_stop = nullptr;

int fail(int status, const std::string& msg) {
  g_error = msg;
  return status;
}

int succeed() {
  g_error.clear();
  return PKV_OK;
}

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

}  // namespace

// The status protocol for the library's other host sources (the cache manager).
namespace pkv {
int host_fail(int status, const std::string& msg) { return fail(status, msg); }
int host_ok() { return succeed(); }
}  // namespace pkv

namespace {

int log2i(int64_t x) {
  int r = 0;
  while ((int64_t{1} << r) < x) ++r;
  return r;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t round256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

int elem_bytes(int32_t dtype) { return dtype == PKV_BF16 ? 2 : 4; }

// Checks shared by both operations: element type, head_dim, block_size, heads, pool geometry.
int check_pool(int32_t dtype, int32_t head_dim, int32_t block_size, int32_t num_kv_heads,
               int64_t num_blocks, int64_t block_stride, int64_t* stride_out) {
  if (dtype != PKV_FP32 && dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "dtype must be PKV_FP32 (0) or PKV_BF16 (1)");
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim must be 64 or 128, got " + std::to_string(head_dim));
  if (!is_pow2(block_size) || block_size < 8 || block_size > 256)
    return fail(PKV_ERR_UNSUPPORTED,
                "block_size must be a power of two in [8, 256], got " + std::to_string(block_size));
  if (num_kv_heads < 1) return fail(PKV_ERR_INVALID_ARG, "num_kv_heads must be >= 1");
  if (num_blocks < 1) return fail(PKV_ERR_INVALID_ARG, "num_blocks must be >= 1");
  if (num_blocks > (int64_t{INT32_MAX} / block_size))
    return fail(PKV_ERR_UNSUPPORTED, "num_blocks * block_size must be < 2^31");
  const int64_t dense = static_cast<int64_t>(block_size) * num_kv_heads * head_dim;
  if (block_stride == 0) block_stride = dense;
  if (block_stride < dense)
    return fail(PKV_ERR_INVALID_ARG, "block_stride is smaller than block_size * num_kv_heads * head_dim");
  if ((block_stride * elem_bytes(dtype)) % 16 != 0)
    return fail(PKV_ERR_INVALID_ARG, "block_stride * element size must be a multiple of 16 bytes");
  *stride_out = block_stride;
  return PKV_OK;
}

struct WsLayout {
  size_t hdr, seq_tiles, tile_rec, tile_q, units, part_ml, part_acc, tok_info, total;
  int64_t tile_cap, unit_cap, prow_cap;
};

// The device picks each sequence's row tile (128 or 256 rows, pkv::tile_kind_for), so the layout bounds the
// tile count with the shorter one: ceil(rows / 128) per sequence at most.  tile_kind 2 (forced) gives the
// tighter bound of 256-row tiles.
WsLayout workspace_layout(int32_t num_seqs, int64_t total_q, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int tile_kind, int64_t partial_rows = pkv::kPartialRowCap) {
  WsLayout w{};
  w.prow_cap = partial_rows;
  const int group = num_q_heads / num_kv_heads;
  const int64_t rt = pkv::tile_rows_of(tile_kind == 2 ? 2 : 1);
  // Each sequence adds at most one partly filled tile.
  w.tile_cap = (total_q * group + rt - 1) / rt + num_seqs;
  // Room for the items, one unit per tile when nothing is split, and a shared-prefix pass (at most about
  // 256 items plus one per prefix tile).
  w.unit_cap = (pkv::kMaxItems + num_kv_heads - 1) / num_kv_heads + 2 * w.tile_cap + 256;
  size_t off = 0;
  w.hdr = off;
  off = round256(off + 16 * sizeof(int));
  w.seq_tiles = off;
  off = round256(off + static_cast<size_t>(num_seqs) * sizeof(int));
  w.tile_rec = off;
  off = round256(off + static_cast<size_t>(w.tile_cap) * 4 * sizeof(int));
  w.tile_q = off;
  off = round256(off + static_cast<size_t>(w.tile_cap) * 2 * sizeof(int));
  w.units = off;
  off = round256(off + static_cast<size_t>(w.unit_cap) * 8 * sizeof(int));
  const size_t part_rows = static_cast<size_t>(partial_rows);
  w.part_ml = off;
  off = round256(off + part_rows * 2 * sizeof(float));
  w.part_acc = off;
  off = round256(off + part_rows * head_dim * sizeof(float));
  w.tok_info = off;
  off = round256(off + static_cast<size_t>(total_q) * 4 * sizeof(int));
  w.total = off;
  return w;
}

int num_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
      cu = 256;
    cached[dev] = cu;
  }
  return cached[dev];
}

int hip_fail(const char* what, hipError_t e) {
  return fail(PKV_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Device scratch of paged_attention_forward_noalloc, in place of a caller's workspace.  Each GPU the
// library runs on holds its own copy until the process ends.  In host code `scratch` only names the
// variable: its device address, per device, comes from hipGetSymbolAddress (scratch_address below) and
// is what the kernels are given.
constexpr size_t kScratchBytes = size_t{PKV_NOALLOC_SCRATCH_BYTES};
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of the current device's scratch, looked up once per device (with that device current).
int scratch_address(void** addr) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  if (dev < 0 || dev >= kMaxDevices) return fail(PKV_ERR_UNSUPPORTED, "device index beyond the library's table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t g = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (g != hipSuccess) return hip_fail("hipGetSymbolAddress(scratch)", g);
    if (p == nullptr) return fail(PKV_ERR_HIP, "hipGetSymbolAddress(scratch) returned a null address");
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return PKV_OK;
}

}  // namespace

namespace {

// Checks paged_kv_write's arguments and fills *p (p->num_tokens == 0: nothing to write).  Launches nothing.
int write_params(const void* k, const void* v, const int32_t* slot_mapping, int64_t num_tokens, void* k_cache,
                 void* v_cache, int64_t num_blocks, int32_t block_size, int64_t block_stride, int32_t num_kv_heads,
                 int32_t head_dim, int32_t dtype, pkv::KvWriteParams* p) {
  if (num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "num_tokens must be >= 0");
  int64_t stride = 0;
  const int rc = check_pool(dtype, head_dim, block_size, num_kv_heads, num_blocks, block_stride, &stride);
  if (rc != PKV_OK) return rc;
  *p = pkv::KvWriteParams{};
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache)
    return fail(PKV_ERR_INVALID_ARG, "null pointer among k, v, slot_mapping, k_cache, v_cache");
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(slot_mapping, 4))
    return fail(PKV_ERR_INVALID_ARG, "k, v, k_cache, v_cache must be 16-byte aligned");
  const int64_t row_bytes = static_cast<int64_t>(num_kv_heads) * head_dim * elem_bytes(dtype);
  const int64_t cpr = row_bytes / 16;
  // The kernel strides over the 16-byte chunks with a 32-bit index: the last stride must not overflow.
  if (num_tokens > (int64_t{INT32_MAX} - pkv::kWriteGridLanes) / (2 * cpr))
    return fail(PKV_ERR_UNSUPPORTED, "num_tokens * row size too large for one call; split the write");
  p->k = k;
  p->v = v;
  p->slot_mapping = slot_mapping;
  p->k_cache = k_cache;
  p->v_cache = v_cache;
  p->num_tokens = static_cast<int>(num_tokens);
  p->chunks_per_row = static_cast<int>(cpr);
  p->block_size_log2 = log2i(block_size);
  p->num_slots = num_blocks * block_size;
  p->block_stride_bytes = stride * elem_bytes(dtype);
  return PKV_OK;
}

}  // namespace

extern "C" {

int paged_kv_abi_version(void) { return kAbiVersion; }

const char* paged_kv_last_error(void) { return g_error.c_str(); }

int paged_kv_write(const void* k, const void* v, const int32_t* slot_mapping, int64_t num_tokens,
                   void* k_cache, void* v_cache, int64_t num_blocks, int32_t block_size,
                   int64_t block_stride, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                   void* stream) {
  pkv::KvWriteParams p{};
  const int rc = write_params(k, v, slot_mapping, num_tokens, k_cache, v_cache, num_blocks, block_size,
                              block_stride, num_kv_heads, head_dim, dtype, &p);
  if (rc != PKV_OK) return rc;
  if (p.num_tokens == 0) return succeed();
  const hipError_t e = pkv::launch_kv_write(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("paged_kv_write launch", e);
  return succeed();
}

int paged_kv_copy_blocks(void* k_cache, void* v_cache, int64_t num_blocks, int32_t block_size,
                         int64_t block_stride, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                         const int32_t* src_blocks, const int32_t* dst_blocks, int32_t num_pairs,
                         void* stream) {
  int64_t stride = 0;
  const int st = check_pool(dtype, head_dim, block_size, num_kv_heads, num_blocks, block_stride, &stride);
  if (st != PKV_OK) return st;
  if (num_pairs < 0) return fail(PKV_ERR_INVALID_ARG, "num_pairs must be >= 0");
  if (num_pairs == 0) return succeed();
  if (num_pairs > 65535) return fail(PKV_ERR_UNSUPPORTED, "at most 65535 pairs per call");
  if (!k_cache || !v_cache || !src_blocks || !dst_blocks)
    return fail(PKV_ERR_INVALID_ARG, "null pointer");
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(PKV_ERR_INVALID_ARG, "caches must be 16-byte aligned");
  pkv::CopyBlocksParams p{};
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.src = src_blocks;
  p.dst = dst_blocks;
  p.num_blocks = num_blocks;
  p.chunks_per_block = static_cast<int64_t>(block_size) * num_kv_heads * head_dim * elem_bytes(dtype) / 16;
  p.block_stride_bytes = stride * elem_bytes(dtype);
  const hipError_t e = pkv::launch_copy_blocks(p, num_pairs, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_ERR_HIP, std::string("copy_blocks launch: ") + hipGetErrorString(e));
  return succeed();
}

size_t paged_attention_workspace_size(int32_t num_seqs, int64_t total_q, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                                      int32_t max_q_len_hint) {
  if (num_seqs < 0 || total_q < 0 || num_kv_heads < 1 || num_q_heads < 1 ||
      num_q_heads % num_kv_heads != 0 || (head_dim != 64 && head_dim != 128) ||
      (dtype != PKV_FP32 && dtype != PKV_BF16)) {
    fail(PKV_ERR_INVALID_ARG, "invalid sizes for paged_attention_workspace_size");
    return 0;
  }
  g_error.clear();
  (void)max_q_len_hint;  // accepted for callers that have it; the device sizes each sequence's tiles itself
  if (dtype == PKV_FP32 || num_seqs == 0 || total_q == 0) return 0;
  return workspace_layout(num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, g_tile_kind).total;
}

}  // extern "C"

namespace {

// Every attention entry point.  `prefix` enables the shared-prefix pass (and the 256-row tiles it runs
// on); its range was checked by the caller.  run_only: the workspace already holds this call's plan (left by
// an earlier call with the same metadata): no planning launch.
int attention_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                   const int32_t* query_start_loc, int32_t num_seqs, int64_t total_q, int32_t num_q_heads,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                   int64_t block_stride, float scale, int32_t dtype, int32_t max_q_len_hint,
                   const pkv::PrefixParams* prefix, void* workspace, size_t workspace_bytes, void* stream,
                   bool noalloc = false, bool run_only = false, const pkv::KvWriteParams* fused_write = nullptr) {
  if (num_seqs < 0 || total_q < 0) return fail(PKV_ERR_INVALID_ARG, "num_seqs and total_q must be >= 0");
  int64_t stride = 0;
  const int rc = check_pool(dtype, head_dim, block_size, num_kv_heads, num_blocks, block_stride, &stride);
  if (rc != PKV_OK) return rc;
  if (num_q_heads < 1 || num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "num_q_heads must be a positive multiple of num_kv_heads");
  if (max_blocks_per_seq < 1) return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq must be >= 1");
  // The plan packs a partition's key count into the upper 30 bits of a 32-bit word.
  if (static_cast<int64_t>(max_blocks_per_seq) * block_size >= (int64_t{1} << 29))
    return fail(PKV_ERR_UNSUPPORTED, "max_blocks_per_seq * block_size must be < 2^29");
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(PKV_ERR_INVALID_ARG, "scale must be finite and positive");
  const int group = num_q_heads / num_kv_heads;
  if (total_q * group > INT32_MAX / 2 || total_q * num_q_heads > INT32_MAX)
    return fail(PKV_ERR_UNSUPPORTED, "total_q too large for one call");
  // A K/V write to do first (fused_write): with the plan when there is one, else on its own.
  const bool write_first = fused_write != nullptr && fused_write->num_tokens > 0;
  if (num_seqs == 0 || total_q == 0) {
    if (write_first) {
      const hipError_t e = pkv::launch_kv_write(*fused_write, static_cast<hipStream_t>(stream));
      if (e != hipSuccess) return hip_fail("paged_kv_write launch", e);
    }
    return succeed();
  }
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start_loc)
    return fail(PKV_ERR_INVALID_ARG,
                "null pointer among out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc");
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(PKV_ERR_INVALID_ARG, "out, q, k_cache, v_cache must be 16-byte aligned");

  pkv::AttnParams p{};
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.query_start_loc = query_start_loc;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = group;
  p.block_size_log2 = log2i(block_size);
  p.num_blocks = num_blocks;
  p.block_stride = stride;
  p.total_q = total_q;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const bool timed = g_ev_start != nullptr && g_ev_stop != nullptr;

  if (dtype == PKV_FP32) {
    if (write_first) {
      const hipError_t e = pkv::launch_kv_write(*fused_write, st);
      if (e != hipSuccess) return hip_fail("paged_kv_write launch", e);
    }
    if (timed) hipEventRecord(g_ev_start, st);
    hipError_t e = pkv::launch_attention_fp32(p, head_dim, st);
    if (e != hipSuccess) return hip_fail("fp32 attention launch", e);
    if (timed) hipEventRecord(g_ev_stop, st);
    return succeed();
  }

  // Each sequence's tile kind is chosen on the device from its own q_len, unless tuning forces one.  A
  // q-length bound that puts every sequence's rows in one 128-row tile lets the call plan 128-row tiles
  // throughout and run the kernel build with only the 16-row body (a wrong bound only costs speed: longer
  // sequences then take several 128-row tiles).  A call with a shared-prefix pass always runs the build with
  // both bodies: the prefix sequence's units are 256-row tiles whatever the members' kind.
  const bool narrow_only = !prefix && (g_tile_kind == 1 ||
                                       (g_tile_kind == 0 && max_q_len_hint > 0 &&
                                        static_cast<int64_t>(max_q_len_hint) * group <= pkv::tile_rows_of(1)));
  const int tile_kind = narrow_only ? 1 : g_tile_kind;
  WsLayout w = workspace_layout(num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, tile_kind);
  if (noalloc) {
    // The library's scratch: the per-call records must fit; the rest holds as many partial rows as it
    // can (fewer partial rows only make the plan split long contexts into fewer partitions).
    const WsLayout fixed = workspace_layout(num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, tile_kind, 0);
    if (fixed.total + 512 > kScratchBytes)
      return fail(PKV_ERR_UNSUPPORTED, "paged_attention_forward_noalloc: this call's work records need " +
                                           std::to_string(fixed.total) + " bytes, more than the " +
                                           std::to_string(kScratchBytes) + "-byte scratch; use "
                                           "paged_attention_forward with a workspace");
    const int64_t rows = static_cast<int64_t>((kScratchBytes - fixed.total - 512) / (8 + 4 * head_dim));
    w = workspace_layout(num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, tile_kind,
                         rows < pkv::kPartialRowCap ? rows : pkv::kPartialRowCap);
    const int st = scratch_address(&workspace);
    if (st != PKV_OK) return st;
    workspace_bytes = kScratchBytes;
  }
  if (!workspace || workspace_bytes < w.total)
    return fail(PKV_ERR_WORKSPACE, "workspace needs " + std::to_string(w.total) + " bytes, got " +
                                       std::to_string(workspace_bytes));
  if (!aligned(workspace, 256)) return fail(PKV_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  pkv::PlanBuffers b{};
  b.hdr = reinterpret_cast<int*>(ws + w.hdr);
  b.seq_tiles = reinterpret_cast<int*>(ws + w.seq_tiles);
  b.tile_rec = reinterpret_cast<int4*>(ws + w.tile_rec);
  b.tile_q = reinterpret_cast<int2*>(ws + w.tile_q);
  b.units = reinterpret_cast<int4*>(ws + w.units);
  b.part_ml = reinterpret_cast<float2*>(ws + w.part_ml);
  b.part_acc = reinterpret_cast<float*>(ws + w.part_acc);
  b.tok_info = reinterpret_cast<int4*>(ws + w.tok_info);
  p.buf = b;
  p.tile_kind = tile_kind;
  // Signature of this call's shape (plan header words kHdrSig0..2): everything the plan's records and the
  // workspace layout depend on besides the metadata's contents.  A run on an existing plan checks it on the
  // device (FNV-1a over the shape words).
  uint32_t h = 2166136261u;
  for (const int64_t v : {static_cast<int64_t>(num_q_heads), static_cast<int64_t>(num_kv_heads),
                          static_cast<int64_t>(head_dim), static_cast<int64_t>(block_size),
                          static_cast<int64_t>(max_blocks_per_seq), static_cast<int64_t>(tile_kind),
                          static_cast<int64_t>(narrow_only), w.tile_cap, w.unit_cap, w.prow_cap,
                          static_cast<int64_t>(prefix ? prefix->begin : -1),
                          static_cast<int64_t>(prefix ? prefix->end : -1),
                          static_cast<int64_t>(prefix ? prefix->tokens : -1)}) {
    for (int byte = 0; byte < 8; ++byte) {
      h ^= static_cast<uint32_t>((v >> (8 * byte)) & 0xff);
      h *= 16777619u;
    }
  }
  p.sig[0] = num_seqs;
  p.sig[1] = static_cast<int>(total_q);
  p.sig[2] = static_cast<int>(h);

  pkv::PlanParams pp{};
  pp.context_lens = context_lens;
  pp.query_start_loc = query_start_loc;
  pp.num_seqs = num_seqs;
  pp.total_q = total_q;
  pp.group = group;
  pp.num_kv_heads = num_kv_heads;
  pp.tile_kind = tile_kind;
  pp.max_context = max_blocks_per_seq * block_size;
  int items = g_target_items > 0 ? g_target_items : pkv::kDefaultItems;
  if (items > pkv::kMaxItems) items = pkv::kMaxItems;
  pp.target_items = items;
  const int64_t grid_wgs = static_cast<int64_t>(num_cus()) * pkv::attention_wgs_per_cu(head_dim, narrow_only);
  pp.min_items = g_target_items > 0 ? 0 : static_cast<int>(2 * grid_wgs);
  pp.forced_partition = g_partition_keys;
  pp.unit_cap = static_cast<int>(w.unit_cap);
  pp.tile_cap = static_cast<int>(w.tile_cap);
  pp.prow_cap = static_cast<int>(w.prow_cap);
  // Sequence s takes ceil(n_s G / 128) tiles at most: in all at most (total_q G + 127 num_seqs) / 128, and
  // with the q-length hint at most num_seqs ceil(hint G / 128).
  pp.tiles_bound = (total_q * group + 127 * static_cast<int64_t>(num_seqs)) / pkv::tile_rows_of(1);
  if (max_q_len_hint > 0)
    pp.tiles_bound = std::min<int64_t>(pp.tiles_bound, static_cast<int64_t>(num_seqs) *
                                           ((static_cast<int64_t>(max_q_len_hint) * group + 127) / 128));
  if (prefix) pp.prefix = *prefix;
  pp.buf = b;
  for (int i = 0; i < 3; ++i) pp.sig[i] = p.sig[i];

  hipError_t e = hipSuccess;
  if (!run_only) {
    e = write_first ? pkv::launch_write_plan(pp, *fused_write, st) : pkv::launch_plan(pp, st);
    if (e != hipSuccess) return hip_fail("plan launch", e);
  }
  int64_t grid = grid_wgs;
  const int64_t max_items = w.unit_cap * num_kv_heads;
  if (grid > max_items) grid = max_items;
  if (timed) hipEventRecord(g_ev_start, st);
  e = pkv::launch_attention(p, head_dim, narrow_only, static_cast<int>(grid), st);
  if (e != hipSuccess) return hip_fail("attention launch", e);
  if (timed) hipEventRecord(g_ev_stop, st);
  e = pkv::launch_split_reduce(p, head_dim, static_cast<int>(w.tile_cap), st);
  if (e != hipSuccess) return hip_fail("split reduce launch", e);
  return succeed();
}

}  // namespace

extern "C" {

int paged_attention_forward(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, const int32_t* query_start_loc,
                            int32_t num_seqs, int64_t total_q, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int64_t num_blocks, int64_t block_stride, float scale, int32_t dtype,
                            int32_t max_q_len_hint, void* workspace, size_t workspace_bytes,
                            void* stream) {
  return attention_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                        query_start_loc, num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_blocks, block_stride, scale, dtype, max_q_len_hint, nullptr, workspace,
                        workspace_bytes, stream);
}

int paged_attention_write_forward(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                                  int64_t num_tokens, void* out, const void* q, void* k_cache, void* v_cache,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, const int32_t* query_start_loc, int32_t num_seqs,
                                  int64_t total_q, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int64_t num_blocks, int64_t block_stride, float scale,
                                  int32_t dtype, int32_t max_q_len_hint, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  pkv::KvWriteParams wp{};
  const int rc = write_params(k_new, v_new, slot_mapping, num_tokens, k_cache, v_cache, num_blocks, block_size,
                              block_stride, num_kv_heads, head_dim, dtype, &wp);
  if (rc != PKV_OK) return rc;
  return attention_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                        query_start_loc, num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_blocks, block_stride, scale, dtype, max_q_len_hint, nullptr, workspace,
                        workspace_bytes, stream, /*noalloc=*/false, /*run_only=*/false, &wp);
}

int paged_attention_run(void* out, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                        const int32_t* query_start_loc, int32_t num_seqs, int64_t total_q, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                        int64_t block_stride, float scale, int32_t dtype, int32_t max_q_len_hint, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return attention_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                        query_start_loc, num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_blocks, block_stride, scale, dtype, max_q_len_hint, nullptr, workspace,
                        workspace_bytes, stream, /*noalloc=*/false, /*run_only=*/true);
}

int paged_attention_forward_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                                    const int32_t* context_lens, const int32_t* query_start_loc,
                                    int32_t num_seqs, int64_t total_q, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                    int64_t num_blocks, int64_t block_stride, float scale, int32_t dtype,
                                    int32_t max_q_len_hint, void* stream) {
  return attention_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                        query_start_loc, num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_blocks, block_stride, scale, dtype, max_q_len_hint, nullptr, nullptr, 0, stream,
                        /*noalloc=*/true);
}

size_t paged_attention_prefix_workspace_size(int32_t num_seqs, int64_t total_q, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim, int32_t dtype) {
  if (num_seqs < 0 || total_q < 0 || num_kv_heads < 1 || num_q_heads < 1 ||
      num_q_heads % num_kv_heads != 0 || (head_dim != 64 && head_dim != 128) ||
      (dtype != PKV_FP32 && dtype != PKV_BF16)) {
    fail(PKV_ERR_INVALID_ARG, "invalid sizes for paged_attention_prefix_workspace_size");
    return 0;
  }
  g_error.clear();
  if (dtype == PKV_FP32 || num_seqs == 0 || total_q == 0) return 0;
  return workspace_layout(num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, g_tile_kind).total;
}

int paged_attention_forward_prefix(void* out, const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens, const int32_t* query_start_loc,
                                   int32_t num_seqs, int64_t total_q, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int64_t num_blocks, int64_t block_stride, float scale, int32_t dtype,
                                   int32_t prefix_begin, int32_t prefix_end, int32_t prefix_tokens,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  if (prefix_begin < 0 || prefix_end < prefix_begin || prefix_end > num_seqs || prefix_tokens < 0)
    return fail(PKV_ERR_INVALID_ARG, "need 0 <= prefix_begin <= prefix_end <= num_seqs and prefix_tokens >= 0");
  if (block_size > 0 && prefix_tokens % block_size != 0)
    return fail(PKV_ERR_INVALID_ARG, "prefix_tokens must be a multiple of block_size");
  if (static_cast<int64_t>(prefix_tokens) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return fail(PKV_ERR_INVALID_ARG, "prefix_tokens exceeds max_blocks_per_seq * block_size");
  const pkv::PrefixParams pre{prefix_begin, prefix_end, prefix_tokens};
  return attention_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                        query_start_loc, num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_blocks, block_stride, scale, dtype, 0, &pre, workspace, workspace_bytes, stream);
}

int paged_attention_run_prefix(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, const int32_t* query_start_loc, int32_t num_seqs,
                               int64_t total_q, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int64_t num_blocks, int64_t block_stride, float scale,
                               int32_t dtype, int32_t prefix_begin, int32_t prefix_end, int32_t prefix_tokens,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (prefix_begin < 0 || prefix_end < prefix_begin || prefix_end > num_seqs || prefix_tokens < 0)
    return fail(PKV_ERR_INVALID_ARG, "need 0 <= prefix_begin <= prefix_end <= num_seqs and prefix_tokens >= 0");
  if (block_size > 0 && prefix_tokens % block_size != 0)
    return fail(PKV_ERR_INVALID_ARG, "prefix_tokens must be a multiple of block_size");
  if (static_cast<int64_t>(prefix_tokens) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return fail(PKV_ERR_INVALID_ARG, "prefix_tokens exceeds max_blocks_per_seq * block_size");
  const pkv::PrefixParams pre{prefix_begin, prefix_end, prefix_tokens};
  return attention_impl(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                        query_start_loc, num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, block_size,
                        num_blocks, block_stride, scale, dtype, 0, &pre, workspace, workspace_bytes, stream,
                        /*noalloc=*/false, /*run_only=*/true);
}

int paged_attention_set_tuning(int32_t partition_keys, int32_t target_items, int32_t tile_kind) {
  if (partition_keys < 0 || target_items < 0 || tile_kind < 0 || tile_kind > 2)
    return fail(PKV_ERR_INVALID_ARG, "tuning values must be >= 0 and tile_kind in {0, 1, 2}");
  if (target_items > pkv::kMaxItems)
    return fail(PKV_ERR_INVALID_ARG, "target_items must be <= " + std::to_string(pkv::kMaxItems));
  g_partition_keys = partition_keys;
  g_target_items = target_items;
  g_tile_kind = tile_kind;
  return succeed();
}

int paged_attention_set_profile_events(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(PKV_ERR_INVALID_ARG, "pass both events or neither");
  g_ev_start = static_cast<hipEvent_t>(start_event);
  g_ev_stop = static_cast<hipEvent_t>(stop_event);
  return succeed();
}

}  // extern "C"
