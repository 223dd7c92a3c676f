// C ABI of libpa: argument validation on the host, then kernel launches on the
// caller's stream.  Nothing here allocates, synchronises or reads device
// memory.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "../../include/pa.h"
#include "pa_kernels.h"

namespace {

thread_local char g_err[512] = "no error";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

int elem_size(int dt) { return dt == PA_F32 ? 4 : dt == PA_BF16 ? 2 : dt == PA_INT8 ? 1 : 0; }

constexpr long kMaxGrid = 2147483647L;
constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

unsigned* status_ptr();

struct SplitPlan {
  int split_tokens = 0;
  int max_pieces = 1;
  size_t o_bytes = 0;
  size_t lse_bytes = 0;
  size_t total() const { return max_pieces > 1 ? o_bytes + lse_bytes : 0; }
};

// Which kernel serves a call.  The matrix cores take every verify call and
// every int8 cache; a bf16 decode call goes there too from groups of 4 query
// heads up (measured: at G = 2 the vector-ALU kernel is ~5 % faster, at G = 6
// the matrix-core one ~15 %).  fp32 decode stays on the vector ALUs.
#ifndef PA_ROWS_MIN_GROUP
#define PA_ROWS_MIN_GROUP 4
#endif
bool rows_kernel(int T, int G, int kv_dtype) {
  return T > 1 || kv_dtype == PA_INT8 || (kv_dtype == PA_BF16 && G >= PA_ROWS_MIN_GROUP);
}

// Piece length for split_tokens = 0.  It depends on the shape only, never on
// the batch.  Pieces trade parallelism (more workgroups for few, long
// sequences) against the partial-result traffic and the merge launch; with
// few KV heads a sequence feeds few workgroups, so its context is cut finer.
//  - matrix-core kernel: 1024 positions per KV head, within [2048, 4096].
//  - vector-ALU kernel: 64 positions per KV head, within [128, 512].
int clamp_int(int x, int lo, int hi) { return x < lo ? lo : x > hi ? hi : x; }
int default_split(int T, int q_heads, int kv_heads, int head_dim, int kv_dtype) {
  (void)head_dim;
#ifdef PA_DEFAULT_SPLIT
  return PA_DEFAULT_SPLIT;
#else
  const int kv = kv_heads < 64 ? kv_heads : 64;
  const int G = kv_heads > 0 ? q_heads / kv_heads : 1;
  if (rows_kernel(T, G, kv_dtype)) return clamp_int(1024 * kv, 2048, 4096);
  return clamp_int(64 * kv, 128, 512);
#endif
}

// Validates sizes shared by decode and verify and fills the split plan.
// rows_rule: the call runs on the matrix-core kernel whatever T is (variable-
// length verify), so the default piece length follows that kernel's rule.
int plan_pieces(int num_seqs, int T, int q_heads, int kv_heads, int head_dim,
                int max_context_len, int kv_dtype, int split_tokens, SplitPlan* plan,
                bool rows_rule = false) {
  if (num_seqs < 0 || T < 1 || q_heads <= 0 || kv_heads <= 0 || max_context_len < 0)
    return fail(PA_ERR_INVALID_ARG,
                "invalid sizes: num_seqs=%d num_query_tokens=%d q_heads=%d kv_heads=%d "
                "max_context_len=%d",
                num_seqs, T, q_heads, kv_heads, max_context_len);
  if (q_heads % kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "q_heads (%d) is not a multiple of kv_heads (%d)", q_heads,
                kv_heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d not built (64 or 128)", head_dim);
  if (kv_dtype != PA_F32 && kv_dtype != PA_BF16 && kv_dtype != PA_INT8)
    return fail(PA_ERR_INVALID_ARG, "unknown kv dtype %d", kv_dtype);
  int st = split_tokens == 0
               ? default_split(rows_rule && T < 2 ? 2 : T, q_heads, kv_heads, head_dim, kv_dtype)
               : split_tokens;
  if (st <= 0 || st % pa::kBlockSizeHost != 0 || st > pa::kMaxSplitTokens)
    return fail(PA_ERR_INVALID_ARG, "split_tokens %d must be a multiple of %d in [%d, %d]",
                split_tokens, pa::kBlockSizeHost, pa::kBlockSizeHost, pa::kMaxSplitTokens);
  plan->split_tokens = st;
  plan->max_pieces = max_context_len > 0 ? int((long(max_context_len) + st - 1) / st) : 1;
  const size_t rows = size_t(num_seqs) * T * q_heads;   // each factor < 2^31: fits
  // partial outputs and log-sum-exps must be addressable: rows * pieces *
  // (head_dim + 1) fp32 values (checked by division, so nothing wraps)
  if (rows > 0 && size_t(plan->max_pieces) * (head_dim + 1) * sizeof(float) >
                      (size_t(1) << 62) / rows)
    return fail(PA_ERR_UNSUPPORTED, "workspace for these sizes exceeds 2^62 bytes");
  plan->o_bytes = round_up(rows * plan->max_pieces * head_dim * sizeof(float));
  plan->lse_bytes = round_up(rows * plan->max_pieces * sizeof(float));
  if (long(plan->max_pieces) * num_seqs * kv_heads > kMaxGrid)
    return fail(PA_ERR_UNSUPPORTED, "too many workgroups: pieces * num_seqs * kv_heads > %ld",
                kMaxGrid);
  return PA_OK;
}

// Bytes of a work plan for num_seqs sequences cut into max_pieces pieces of
// split_tokens positions; 0 when the units exceed what one plan orders.
size_t plan_bytes_for(int num_seqs, const SplitPlan& sp) {
  const long units = long(num_seqs) * sp.max_pieces;
  if (units > pa::kMaxPlanUnits) return 0;
  return size_t(pa::kPlanHeader + units * pa::plan_stride(sp.split_tokens)) * sizeof(int32_t);
}

int check_attention_args(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const float* k_scale, const float* v_scale,
                         const int32_t* block_tables, const int32_t* context_lens,
                         int num_seqs, int kv_heads, int block_size, int num_blocks,
                         int max_blocks_per_seq, int max_context_len, float scale, int q_dtype,
                         int kv_dtype, bool no_rows = false) {
  if (block_size != 16) return fail(PA_ERR_UNSUPPORTED, "block_size %d not built (16)", block_size);
  if (num_blocks <= 0 || max_blocks_per_seq <= 0)
    return fail(PA_ERR_INVALID_ARG, "num_blocks (%d) and max_blocks_per_seq (%d) must be > 0",
                num_blocks, max_blocks_per_seq);
  if (long(max_context_len) > long(max_blocks_per_seq) * block_size)
    return fail(PA_ERR_INVALID_ARG, "max_context_len %d exceeds max_blocks_per_seq * block_size",
                max_context_len);
  const bool triple_ok = (q_dtype == PA_F32 && kv_dtype == PA_F32) ||
                         (q_dtype == PA_BF16 && kv_dtype == PA_BF16) ||
                         (q_dtype == PA_BF16 && kv_dtype == PA_INT8);
  if (!triple_ok) {
    if (elem_size(q_dtype) == 0 || q_dtype == PA_INT8)
      return fail(PA_ERR_INVALID_ARG, "invalid q dtype %d", q_dtype);
    return fail(PA_ERR_UNSUPPORTED, "dtype pair q=%d kv=%d not built", q_dtype, kv_dtype);
  }
  if (!isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale is not finite");
  // nothing to read or write: the (empty) arrays may be NULL
  if (num_seqs == 0 || no_rows) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (kv_dtype == PA_INT8 && (!k_scale || !v_scale))
    return fail(PA_ERR_INVALID_ARG, "int8 cache needs k_scale and v_scale");
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(PA_ERR_INVALID_ARG, "out, q and the caches must be 16-byte aligned");
  if (!aligned(block_tables, 4) || !aligned(context_lens, 4) ||
      (k_scale && !aligned(k_scale, 4)) || (v_scale && !aligned(v_scale, 4)))
    return fail(PA_ERR_INVALID_ARG, "misaligned table, length or scale pointer");
  return PA_OK;
}

struct Append {
  const void* key = nullptr;
  const void* value = nullptr;
  const int64_t* slot_mapping = nullptr;
  int in_dtype = -1;   // requantizing write into an int8 cache: PA_F32 / PA_BF16 rows
  bool on = false;
};

// Variable-length verify: packed query rows with per-sequence offsets.
struct Varlen {
  const int32_t* query_start = nullptr;
  int total = 0;
  bool on = false;
};

int run_attention(bool is_verify, void* out, const void* q, const void* k_cache,
                  const void* v_cache, const float* k_scale, const float* v_scale,
                  const int32_t* block_tables, const int32_t* context_lens, int num_seqs, int T,
                  int q_heads, int kv_heads, int head_dim, int block_size, int num_blocks,
                  int max_blocks_per_seq, int max_context_len, float scale, int q_dtype,
                  int kv_dtype, int split_tokens, void* workspace, size_t workspace_bytes,
                  void* stream, const Append& app = Append(), const Varlen& vl = Varlen(),
                  const void* work_plan = nullptr, size_t work_plan_bytes = 0) {
  SplitPlan plan;
  int st = plan_pieces(num_seqs, T, q_heads, kv_heads, head_dim, max_context_len, kv_dtype,
                       split_tokens, &plan, vl.on);
  if (st != PA_OK) return st;
  if (app.on && kv_dtype == PA_INT8 && app.in_dtype < 0)
    return fail(PA_ERR_UNSUPPORTED,
                "append into an int8 cache takes bf16/fp32 rows (pa_decode_append_quant)");
  if (app.on && app.in_dtype >= 0) {
    if (kv_dtype != PA_INT8)
      return fail(PA_ERR_INVALID_ARG, "the requantizing append needs an int8 cache");
    if (app.in_dtype != PA_F32 && app.in_dtype != PA_BF16)
      return fail(PA_ERR_INVALID_ARG, "key/value dtype %d: PA_F32 or PA_BF16", app.in_dtype);
    if (q_heads % kv_heads == 0 && q_heads / kv_heads > 16)
      return fail(PA_ERR_UNSUPPORTED, "the requantizing append takes groups of at most 16 heads");
  }
  if (vl.on && (vl.total < 0 || long(vl.total) > long(num_seqs) * T))
    return fail(PA_ERR_INVALID_ARG,
                "total_query_tokens %d must be in [0, num_seqs * max_query_tokens = %ld]",
                vl.total, long(num_seqs) * T);
  st = check_attention_args(out, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                            context_lens, num_seqs, kv_heads, block_size, num_blocks,
                            max_blocks_per_seq, max_context_len, scale, q_dtype, kv_dtype,
                            vl.on && vl.total == 0);
  if (st != PA_OK) return st;
  const int G = q_heads / kv_heads;
  // Verify calls with more query rows per (sequence, KV head) than the
  // matrix-core decode kernel's row tiles hold run on the prefill kernel, which
  // has no row limit (and no pieces: each sequence's whole context in one
  // workgroup per 128 rows).
  const bool verify_on_prefill = is_verify && !pa::rows_supported(q_dtype, kv_dtype, head_dim, G, T);
  if (is_verify) {
    if (verify_on_prefill && !pa::prefill_supported(q_dtype, kv_dtype, head_dim))
      return fail(PA_ERR_UNSUPPORTED,
                  "verify not built for q=%d kv=%d head_dim=%d group=%d tokens=%d", q_dtype,
                  kv_dtype, head_dim, G, T);
    if (verify_on_prefill && (long(T) * q_heads > 2147483647L ||
                              long(num_seqs) * kv_heads *
                                      ((long(T) * G + pa::prefill_rows_per_workgroup() - 1) /
                                       pa::prefill_rows_per_workgroup()) > kMaxGrid))
      return fail(PA_ERR_UNSUPPORTED, "too many query rows or workgroups");
  } else if (!pa::decode_group_supported(G)) {
    return fail(PA_ERR_UNSUPPORTED, "group size %d not built (1..8 or 16)", G);
  }
  if (app.on) {
    if (num_seqs > 0 && (!app.key || !app.value || !app.slot_mapping))
      return fail(PA_ERR_INVALID_ARG, "null key, value or slot_mapping");
    if (!aligned(app.key, 16) || !aligned(app.value, 16) || !aligned(app.slot_mapping, 8))
      return fail(PA_ERR_INVALID_ARG, "misaligned key, value or slot_mapping");
  }
  if (vl.on && num_seqs > 0 && (!vl.query_start || !aligned(vl.query_start, 4)))
    return fail(PA_ERR_INVALID_ARG, "query_start must be a 4-byte aligned pointer");
  if (vl.on && vl.total == 0) return PA_OK;
  if (work_plan) {
    const size_t pb = plan_bytes_for(num_seqs, plan);
    if (pb == 0)
      return fail(PA_ERR_UNSUPPORTED, "a work plan orders at most %d (sequence, piece) units",
                  pa::kMaxPlanUnits);
    if (work_plan_bytes < pb || !aligned(work_plan, 16))
      return fail(PA_ERR_INVALID_ARG,
                  "work plan of %zu bytes (16-byte aligned) needed for these sizes, got %zu", pb,
                  work_plan_bytes);
  }
  if (num_seqs == 0) return PA_OK;
  const size_t need = verify_on_prefill ? 0 : plan.total();
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, kAlign)))
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes (256-byte aligned) needed, got %zu",
                need, workspace ? workspace_bytes : size_t(0));

  pa::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  char* ws = static_cast<char*>(workspace);
  a.part_lse = need ? reinterpret_cast<float*>(ws) : nullptr;
  a.part_o = need ? reinterpret_cast<float*>(ws + plan.lse_bytes) : nullptr;
  a.num_seqs = num_seqs;
  a.num_query_tokens = T;
  a.q_heads = q_heads;
  a.kv_heads = kv_heads;
  a.head_dim = head_dim;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.split_tokens = plan.split_tokens;
  a.max_pieces = plan.max_pieces;
  a.scale = scale;
  a.q_dtype = q_dtype;
  a.kv_dtype = kv_dtype;
  hipStream_t s = static_cast<hipStream_t>(stream);
  a.new_k = app.key;
  a.new_v = app.value;
  a.slot_mapping = app.slot_mapping;
  a.new_dtype = app.in_dtype == PA_F32 ? pa::kF32 : pa::kBF16;
  a.query_start = vl.on ? vl.query_start : nullptr;
  a.plan = static_cast<const int32_t*>(work_plan);
  a.check_status = status_ptr();
  a.total_query_tokens = vl.on ? vl.total : num_seqs * T;
  hipError_t e = hipSuccess;
  if (verify_on_prefill) {
    a.plan = nullptr;   // a decode-kernel plan orders other units
    a.part_o = a.part_lse = nullptr;
    a.split_tokens = 0;
    a.max_pieces = 1;
    e = pa::launch_prefill(a, s);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "verify launch failed: %s", hipGetErrorString(e));
    return PA_OK;
  }
  // Verify calls, decode over an int8 cache and bf16 decode with large groups
  // run on the matrix cores; both kernels take the fused cache write (bf16 and
  // fp32 caches; int8 append was refused above).
  const bool rows = vl.on || rows_kernel(T, G, kv_dtype);
  e = rows ? pa::launch_rows_pass1(a, s) : pa::launch_decode_pass1(a, app.on, s);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "pass-1 launch failed: %s", hipGetErrorString(e));
  if (plan.max_pieces > 1) {
    pa::MergeArgs m{};
    m.out = out;
    m.part_o = a.part_o;
    m.part_lse = a.part_lse;
    m.context_lens = context_lens;
    m.query_start = a.query_start;
    m.num_seqs = num_seqs;
    m.q_heads = q_heads;
    m.rows_per_seq = T * q_heads;
    m.num_rows = vl.on ? vl.total * q_heads : num_seqs * m.rows_per_seq;
    m.max_pieces = plan.max_pieces;
    m.split_tokens = plan.split_tokens;
    m.max_len_clamp = max_blocks_per_seq * block_size;
    m.head_dim = head_dim;
    m.out_dtype = q_dtype;
    e = pa::launch_merge(m, s);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "merge launch failed: %s", hipGetErrorString(e));
  }
  return PA_OK;
}

}  // namespace

namespace {

// The fixed device array behind pa_decode_noalloc: the split-K partials of a
// call live here instead of in a caller workspace.  Each GPU the library runs
// on holds its own copy until the process ends.  In host code `scratch` only
// names the symbol; its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and that pointer is what
// the kernels receive.
__device__ __align__(256) char scratch[PA_NOALLOC_SCRATCH_BYTES];

#if PA_DEVICE_CHECKS
// The device-check status word of a debug build (one per GPU).
__device__ unsigned check_status_word;
#endif

constexpr int kMaxDevices = 64;
std::mutex g_symbol_mu;
void* g_scratch_ptr[kMaxDevices] = {};
void* g_status_ptr[kMaxDevices] = {};

// Device address of one of this file's device symbols on the current device,
// looked up once per device (with that device current) and cached in
// cache[device].
int symbol_ptr(const void* symbol, void** cache, const char* what, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_symbol_mu);
  if (!cache[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, symbol);
    if (e != hipSuccess || !p)
      return fail(PA_ERR_HIP, "%s address on device %d: %s", what, dev, hipGetErrorString(e));
    cache[dev] = p;
  }
  *out = cache[dev];
  return PA_OK;
}

int scratch_ptr(void** out) {
  return symbol_ptr(HIP_SYMBOL(scratch), g_scratch_ptr, "scratch array", out);
}

// The status word the kernels of a debug build report to (nullptr in release
// builds, whose kernels check nothing).
unsigned* status_ptr() {
#if PA_DEVICE_CHECKS
  void* p = nullptr;
  return symbol_ptr(&check_status_word, g_status_ptr, "check status word", &p) == PA_OK
             ? static_cast<unsigned*>(p)
             : nullptr;
#else
  return nullptr;
#endif
}

}  // namespace

extern "C" {

int pa_version(void) { return 100; }

int pa_device_check_status(unsigned* flags, int clear) {
  if (!flags) return fail(PA_ERR_INVALID_ARG, "null flags pointer");
  *flags = 0;
#if PA_DEVICE_CHECKS
  void* p = nullptr;
  int st = symbol_ptr(&check_status_word, g_status_ptr, "check status word", &p);
  if (st != PA_OK) return st;
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(flags, p, sizeof(unsigned), hipMemcpyDeviceToHost);
  if (e == hipSuccess && clear) {
    const unsigned zero = 0;
    e = hipMemcpy(p, &zero, sizeof(unsigned), hipMemcpyHostToDevice);
  }
  if (e != hipSuccess) return fail(PA_ERR_HIP, "reading the check status word: %s", hipGetErrorString(e));
  return PA_OK;
#else
  (void)clear;
  return fail(PA_ERR_UNSUPPORTED, "device checks are not built into this library (libpa_debug.so has them)");
#endif
}

const char* pa_last_error(void) { return g_err; }

int pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                         const int64_t* slot_mapping, int num_tokens, int kv_heads,
                         int head_dim, int num_blocks, int block_size, int kv_dtype,
                         void* stream) {
  if (num_tokens < 0 || kv_heads <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "invalid sizes: num_tokens=%d kv_heads=%d num_blocks=%d",
                num_tokens, kv_heads, num_blocks);
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d not built (64 or 128)", head_dim);
  if (block_size != 16) return fail(PA_ERR_UNSUPPORTED, "block_size %d not built (16)", block_size);
  if (kv_dtype != PA_F32 && kv_dtype != PA_BF16 && kv_dtype != PA_INT8)
    return fail(PA_ERR_INVALID_ARG, "unknown kv dtype %d", kv_dtype);
  if (num_tokens == 0) return PA_OK;
  // 16-byte chunks of all rows (each factor below 2^31, so no product overflows)
  if (long(num_tokens) * kv_heads > kMaxGrid / (head_dim * elem_size(kv_dtype) / 16))
    return fail(PA_ERR_UNSUPPORTED, "num_tokens * kv_heads * head_dim too large");
  if (!key || !value || !k_cache || !v_cache || !slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(slot_mapping, 8))
    return fail(PA_ERR_INVALID_ARG, "misaligned pointer argument");
  pa::CacheArgs a{key, value, k_cache, v_cache, slot_mapping, num_tokens, kv_heads, num_blocks,
                  head_dim * elem_size(kv_dtype), status_ptr()};
  hipError_t e = pa::launch_reshape_and_cache(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "cache write launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

int pa_reshape_and_cache_quant(const void* key, const void* value, int8_t* k_cache,
                               int8_t* v_cache, float* k_scale, float* v_scale,
                               const int64_t* slot_mapping, int num_tokens, int kv_heads,
                               int head_dim, int num_blocks, int block_size, int in_dtype,
                               void* stream) {
  if (num_tokens < 0 || kv_heads <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "invalid sizes: num_tokens=%d kv_heads=%d num_blocks=%d",
                num_tokens, kv_heads, num_blocks);
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d not built (64 or 128)", head_dim);
  if (block_size != 16) return fail(PA_ERR_UNSUPPORTED, "block_size %d not built (16)", block_size);
  if (in_dtype != PA_F32 && in_dtype != PA_BF16)
    return fail(PA_ERR_INVALID_ARG, "key/value dtype %d: PA_F32 or PA_BF16", in_dtype);
  if (long(num_blocks) * block_size >= 2147483647L)
    return fail(PA_ERR_UNSUPPORTED, "num_blocks * block_size must stay below 2^31");
  if (2L * num_tokens * kv_heads > kMaxGrid)
    return fail(PA_ERR_UNSUPPORTED, "num_tokens * kv_heads too large");
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !k_scale || !v_scale || !slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(k_scale, 4) || !aligned(v_scale, 4) ||
      !aligned(slot_mapping, 8))
    return fail(PA_ERR_INVALID_ARG, "misaligned pointer argument");
  pa::QuantCacheArgs a{key, value, k_cache, v_cache, k_scale, v_scale, slot_mapping,
                       num_tokens, kv_heads, num_blocks, head_dim, in_dtype, status_ptr()};
  hipError_t e = pa::launch_reshape_and_cache_quant(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "cache write launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

int pa_default_split_tokens(int num_query_tokens, int q_heads, int kv_heads, int head_dim,
                            int kv_dtype) {
  return default_split(num_query_tokens, q_heads, kv_heads, head_dim, kv_dtype);
}

size_t pa_workspace_size(int num_seqs, int num_query_tokens, int q_heads, int kv_heads,
                         int head_dim, int max_context_len, int kv_dtype, int split_tokens) {
  SplitPlan plan;
  if (plan_pieces(num_seqs, num_query_tokens, q_heads, kv_heads, head_dim, max_context_len,
                  kv_dtype, split_tokens, &plan) != PA_OK)
    return 0;
  return plan.total();
}

int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const float* k_scale, const float* v_scale, const int32_t* block_tables,
              const int32_t* context_lens, int num_seqs, int q_heads, int kv_heads,
              int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
              int max_context_len, float scale, int q_dtype, int kv_dtype, int split_tokens,
              void* workspace, size_t workspace_bytes, void* stream) {
  return run_attention(false, out, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                       context_lens, num_seqs, 1, q_heads, kv_heads, head_dim, block_size,
                       num_blocks, max_blocks_per_seq, max_context_len, scale, q_dtype, kv_dtype,
                       split_tokens, workspace, workspace_bytes, stream);
}

int pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const float* k_scale, const float* v_scale, const int32_t* block_tables,
                      const int32_t* context_lens, int num_seqs, int q_heads, int kv_heads,
                      int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                      int max_context_len, float scale, int q_dtype, int kv_dtype,
                      int split_tokens, void* stream) {
  SplitPlan plan;
  int st = plan_pieces(num_seqs, 1, q_heads, kv_heads, head_dim, max_context_len, kv_dtype,
                       split_tokens, &plan);
  if (st != PA_OK) return st;
  const size_t need = plan.total();
  if (need > size_t(PA_NOALLOC_SCRATCH_BYTES))
    return fail(PA_ERR_WORKSPACE,
                "these sizes need %zu bytes of partials; the fixed scratch array holds %zu "
                "(use pa_decode with a workspace, or a longer split_tokens)",
                need, size_t(PA_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  if (need > 0 && num_seqs > 0) {
    st = scratch_ptr(&ws);
    if (st != PA_OK) return st;
  }
  return run_attention(false, out, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                       context_lens, num_seqs, 1, q_heads, kv_heads, head_dim, block_size,
                       num_blocks, max_blocks_per_seq, max_context_len, scale, q_dtype, kv_dtype,
                       split_tokens, ws, ws ? size_t(PA_NOALLOC_SCRATCH_BYTES) : 0, stream);
}

int pa_decode_append(void* out, const void* q, const void* key, const void* value,
                     void* k_cache, void* v_cache, const int64_t* slot_mapping,
                     const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                     int q_heads, int kv_heads, int head_dim, int block_size, int num_blocks,
                     int max_blocks_per_seq, int max_context_len, float scale, int q_dtype,
                     int kv_dtype, int split_tokens, void* workspace, size_t workspace_bytes,
                     void* stream) {
  Append app;
  app.key = key;
  app.value = value;
  app.slot_mapping = slot_mapping;
  app.on = true;
  return run_attention(false, out, q, k_cache, v_cache, nullptr, nullptr, block_tables,
                       context_lens, num_seqs, 1, q_heads, kv_heads, head_dim, block_size,
                       num_blocks, max_blocks_per_seq, max_context_len, scale, q_dtype, kv_dtype,
                       split_tokens, workspace, workspace_bytes, stream, app);
}

int pa_decode_append_quant(void* out, const void* q, const void* key, const void* value,
                           int in_dtype, int8_t* k_cache, int8_t* v_cache, float* k_scale,
                           float* v_scale, const int64_t* slot_mapping,
                           const int32_t* block_tables, const int32_t* context_lens,
                           int num_seqs, int q_heads, int kv_heads, int head_dim, int block_size,
                           int num_blocks, int max_blocks_per_seq, int max_context_len,
                           float scale, int split_tokens, void* workspace,
                           size_t workspace_bytes, void* stream) {
  Append app;
  app.key = key;
  app.value = value;
  app.slot_mapping = slot_mapping;
  app.in_dtype = in_dtype;
  app.on = true;
  return run_attention(false, out, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                       context_lens, num_seqs, 1, q_heads, kv_heads, head_dim, block_size,
                       num_blocks, max_blocks_per_seq, max_context_len, scale, PA_BF16, PA_INT8,
                       split_tokens, workspace, workspace_bytes, stream, app);
}

int pa_verify(void* out, const void* q, const void* k_cache, const void* v_cache,
              const float* k_scale, const float* v_scale, const int32_t* block_tables,
              const int32_t* context_lens, int num_seqs, int num_query_tokens, int q_heads,
              int kv_heads, int head_dim, int block_size, int num_blocks,
              int max_blocks_per_seq, int max_context_len, float scale, int q_dtype,
              int kv_dtype, int split_tokens, void* workspace, size_t workspace_bytes,
              void* stream) {
  return run_attention(true, out, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                       context_lens, num_seqs, num_query_tokens, q_heads, kv_heads, head_dim,
                       block_size, num_blocks, max_blocks_per_seq, max_context_len, scale,
                       q_dtype, kv_dtype, split_tokens, workspace, workspace_bytes, stream);
}

size_t pa_plan_size(int num_seqs, int num_query_tokens, int q_heads, int kv_heads,
                    int head_dim, int max_context_len, int kv_dtype, int split_tokens) {
  SplitPlan sp;
  if (plan_pieces(num_seqs, num_query_tokens, q_heads, kv_heads, head_dim, max_context_len,
                  kv_dtype, split_tokens, &sp) != PA_OK)
    return 0;
  const size_t pb = plan_bytes_for(num_seqs, sp);
  if (pb == 0)
    fail(PA_ERR_UNSUPPORTED, "a work plan orders at most %d (sequence, piece) units",
         pa::kMaxPlanUnits);
  return pb;
}

int pa_plan(const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
            int num_query_tokens, int q_heads, int kv_heads, int head_dim,
            int max_blocks_per_seq, int max_context_len, int kv_dtype, int split_tokens,
            void* plan, size_t plan_bytes, void* stream) {
  SplitPlan sp;
  int st = plan_pieces(num_seqs, num_query_tokens, q_heads, kv_heads, head_dim,
                       max_context_len, kv_dtype, split_tokens, &sp);
  if (st != PA_OK) return st;
  if (max_blocks_per_seq <= 0 || long(max_context_len) > long(max_blocks_per_seq) * 16)
    return fail(PA_ERR_INVALID_ARG,
                "max_blocks_per_seq %d must be > 0 and cover max_context_len %d",
                max_blocks_per_seq, max_context_len);
  const size_t pb = plan_bytes_for(num_seqs, sp);
  if (pb == 0)
    return fail(PA_ERR_UNSUPPORTED, "a work plan orders at most %d (sequence, piece) units",
                pa::kMaxPlanUnits);
  if (!plan || plan_bytes < pb || !aligned(plan, 16))
    return fail(PA_ERR_INVALID_ARG,
                "work plan of %zu bytes (16-byte aligned) needed for these sizes, got %zu", pb,
                plan ? plan_bytes : size_t(0));
  if (num_seqs > 0 && (!block_tables || !context_lens))
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(block_tables, 4) || !aligned(context_lens, 4))
    return fail(PA_ERR_INVALID_ARG, "misaligned table or length pointer");
  // Snake rounds where the kernel that will read the plan keeps several
  // workgroups per CU: one round is one workgroup per CU, i.e. CUs / kv_heads
  // units (a unit's kv_heads workgroups are consecutive).
  const int G = q_heads / kv_heads;
  const int resident = rows_kernel(num_query_tokens, G, kv_dtype)
                           ? pa::rows_pass1_resident(kv_dtype, head_dim, num_query_tokens * G)
                           : pa::decode_pass1_resident(kv_dtype == PA_F32 ? PA_F32 : PA_BF16,
                                                       kv_dtype, head_dim, G);
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 0;
  const int snake_units = resident >= 2 && cus > 0 ? (cus + kv_heads - 1) / kv_heads : 0;
  pa::PlanArgs a{block_tables, context_lens, static_cast<int32_t*>(plan), num_seqs,
                 max_blocks_per_seq, sp.max_pieces, sp.split_tokens, snake_units, resident};
  hipError_t e = pa::launch_plan(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "plan launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

int pa_decode_planned(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const float* k_scale, const float* v_scale, const int32_t* block_tables,
                      const int32_t* context_lens, int num_seqs, int q_heads, int kv_heads,
                      int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                      int max_context_len, float scale, int q_dtype, int kv_dtype,
                      int split_tokens, void* workspace, size_t workspace_bytes,
                      const void* plan, size_t plan_bytes, void* stream) {
  if (!plan) return fail(PA_ERR_INVALID_ARG, "null work plan");
  return run_attention(false, out, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                       context_lens, num_seqs, 1, q_heads, kv_heads, head_dim, block_size,
                       num_blocks, max_blocks_per_seq, max_context_len, scale, q_dtype, kv_dtype,
                       split_tokens, workspace, workspace_bytes, stream, Append(), Varlen(),
                       plan, plan_bytes);
}

int pa_decode_append_planned(void* out, const void* q, const void* key, const void* value,
                             void* k_cache, void* v_cache, const int64_t* slot_mapping,
                             const int32_t* block_tables, const int32_t* context_lens,
                             int num_seqs, int q_heads, int kv_heads, int head_dim,
                             int block_size, int num_blocks, int max_blocks_per_seq,
                             int max_context_len, float scale, int q_dtype, int kv_dtype,
                             int split_tokens, void* workspace, size_t workspace_bytes,
                             const void* plan, size_t plan_bytes, void* stream) {
  if (!plan) return fail(PA_ERR_INVALID_ARG, "null work plan");
  Append app;
  app.key = key;
  app.value = value;
  app.slot_mapping = slot_mapping;
  app.on = true;
  return run_attention(false, out, q, k_cache, v_cache, nullptr, nullptr, block_tables,
                       context_lens, num_seqs, 1, q_heads, kv_heads, head_dim, block_size,
                       num_blocks, max_blocks_per_seq, max_context_len, scale, q_dtype, kv_dtype,
                       split_tokens, workspace, workspace_bytes, stream, app, Varlen(), plan,
                       plan_bytes);
}

int pa_decode_append_quant_planned(void* out, const void* q, const void* key,
                                   const void* value, int in_dtype, int8_t* k_cache,
                                   int8_t* v_cache, float* k_scale, float* v_scale,
                                   const int64_t* slot_mapping, const int32_t* block_tables,
                                   const int32_t* context_lens, int num_seqs, int q_heads,
                                   int kv_heads, int head_dim, int block_size, int num_blocks,
                                   int max_blocks_per_seq, int max_context_len, float scale,
                                   int split_tokens, void* workspace, size_t workspace_bytes,
                                   const void* plan, size_t plan_bytes, void* stream) {
  if (!plan) return fail(PA_ERR_INVALID_ARG, "null work plan");
  Append app;
  app.key = key;
  app.value = value;
  app.slot_mapping = slot_mapping;
  app.in_dtype = in_dtype;
  app.on = true;
  return run_attention(false, out, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                       context_lens, num_seqs, 1, q_heads, kv_heads, head_dim, block_size,
                       num_blocks, max_blocks_per_seq, max_context_len, scale, PA_BF16, PA_INT8,
                       split_tokens, workspace, workspace_bytes, stream, app, Varlen(), plan,
                       plan_bytes);
}

int pa_verify_planned(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const float* k_scale, const float* v_scale, const int32_t* block_tables,
                      const int32_t* context_lens, int num_seqs, int num_query_tokens,
                      int q_heads, int kv_heads, int head_dim, int block_size, int num_blocks,
                      int max_blocks_per_seq, int max_context_len, float scale, int q_dtype,
                      int kv_dtype, int split_tokens, void* workspace, size_t workspace_bytes,
                      const void* plan, size_t plan_bytes, void* stream) {
  if (!plan) return fail(PA_ERR_INVALID_ARG, "null work plan");
  return run_attention(true, out, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                       context_lens, num_seqs, num_query_tokens, q_heads, kv_heads, head_dim,
                       block_size, num_blocks, max_blocks_per_seq, max_context_len, scale,
                       q_dtype, kv_dtype, split_tokens, workspace, workspace_bytes, stream,
                       Append(), Varlen(), plan, plan_bytes);
}

}  // extern "C"

namespace {

// Prefill plan bytes for these sizes (0 past kMaxPlanUnits units).
size_t prefill_plan_bytes(int num_seqs, int max_query_tokens, int q_heads, int kv_heads) {
  if (num_seqs < 0 || max_query_tokens < 1 || q_heads <= 0 || kv_heads <= 0 ||
      q_heads % kv_heads != 0)
    return 0;
  const long rows = long(max_query_tokens) * (q_heads / kv_heads);
  const long per_wg = pa::prefill_rows_per_workgroup();
  const long units = long(num_seqs) * ((rows + per_wg - 1) / per_wg);
  if (units > pa::kMaxPlanUnits) return 0;
  return size_t(pa::kPlanHeader + units * pa::kPrefillPlanRow) * sizeof(int32_t);
}

int run_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                const float* k_scale, const float* v_scale, const int32_t* block_tables,
                const int32_t* context_lens, const int32_t* query_start, int num_seqs,
                int total_query_tokens, int max_query_tokens, int q_heads, int kv_heads,
                int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                int max_context_len, float scale, int q_dtype, int kv_dtype, void* stream,
                const void* plan, size_t plan_bytes) {
  if (num_seqs < 0 || max_query_tokens < 1 || q_heads <= 0 || kv_heads <= 0 ||
      max_context_len < 0)
    return fail(PA_ERR_INVALID_ARG,
                "invalid sizes: num_seqs=%d max_query_tokens=%d q_heads=%d kv_heads=%d "
                "max_context_len=%d",
                num_seqs, max_query_tokens, q_heads, kv_heads, max_context_len);
  if (q_heads % kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "q_heads (%d) is not a multiple of kv_heads (%d)", q_heads,
                kv_heads);
  if (!pa::prefill_supported(q_dtype, kv_dtype, head_dim))
    return fail(PA_ERR_UNSUPPORTED, "prefill not built for q=%d kv=%d head_dim=%d", q_dtype,
                kv_dtype, head_dim);
  if (total_query_tokens < 0 || long(total_query_tokens) > long(num_seqs) * max_query_tokens)
    return fail(PA_ERR_INVALID_ARG,
                "total_query_tokens %d must be in [0, num_seqs * max_query_tokens = %ld]",
                total_query_tokens, long(num_seqs) * max_query_tokens);
  int st = check_attention_args(out, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                                context_lens, num_seqs, kv_heads, block_size, num_blocks,
                                max_blocks_per_seq, max_context_len, scale, q_dtype, kv_dtype,
                                total_query_tokens == 0);
  if (st != PA_OK) return st;
  const int G = q_heads / kv_heads;
  const long rows = long(max_query_tokens) * G;
  const long per_wg = pa::prefill_rows_per_workgroup();
  const long tiles = (rows + per_wg - 1) / per_wg;
  if (rows > 2147483647L || long(total_query_tokens) * q_heads > 2147483647L ||
      tiles * num_seqs * kv_heads > kMaxGrid)
    return fail(PA_ERR_UNSUPPORTED, "too many query rows or workgroups");
  if (plan) {
    const size_t pb = prefill_plan_bytes(num_seqs, max_query_tokens, q_heads, kv_heads);
    if (pb == 0)
      return fail(PA_ERR_UNSUPPORTED, "a prefill plan orders at most %d (sequence, row tile) units",
                  pa::kMaxPlanUnits);
    if (plan_bytes < pb || !aligned(plan, 16))
      return fail(PA_ERR_INVALID_ARG,
                  "prefill plan of %zu bytes (16-byte aligned) needed for these sizes, got %zu", pb,
                  plan_bytes);
  }
  if (num_seqs == 0 || total_query_tokens == 0) return PA_OK;
  if (!query_start || !aligned(query_start, 4))
    return fail(PA_ERR_INVALID_ARG, "query_start must be a 4-byte aligned pointer");
  pa::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.total_query_tokens = total_query_tokens;
  a.num_seqs = num_seqs;
  a.num_query_tokens = max_query_tokens;
  a.q_heads = q_heads;
  a.kv_heads = kv_heads;
  a.head_dim = head_dim;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.scale = scale;
  a.q_dtype = q_dtype;
  a.kv_dtype = kv_dtype;
  a.plan = static_cast<const int32_t*>(plan);
  a.check_status = status_ptr();
  hipError_t e = pa::launch_prefill(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
               const float* k_scale, const float* v_scale, const int32_t* block_tables,
               const int32_t* context_lens, const int32_t* query_start, int num_seqs,
               int total_query_tokens, int max_query_tokens, int q_heads, int kv_heads,
               int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
               int max_context_len, float scale, int q_dtype, int kv_dtype, void* stream) {
  return run_prefill(out, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                     query_start, num_seqs, total_query_tokens, max_query_tokens, q_heads,
                     kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                     max_context_len, scale, q_dtype, kv_dtype, stream, nullptr, 0);
}

size_t pa_prefill_plan_size(int num_seqs, int max_query_tokens, int q_heads, int kv_heads) {
  const size_t pb = prefill_plan_bytes(num_seqs, max_query_tokens, q_heads, kv_heads);
  if (pb == 0) fail(PA_ERR_INVALID_ARG, "invalid sizes or more than %d units", pa::kMaxPlanUnits);
  return pb;
}

int pa_prefill_plan(const int32_t* context_lens, const int32_t* query_start, int num_seqs,
                    int total_query_tokens, int max_query_tokens, int q_heads, int kv_heads,
                    int max_blocks_per_seq, void* plan, size_t plan_bytes, void* stream) {
  if (num_seqs < 0 || max_query_tokens < 1 || q_heads <= 0 || kv_heads <= 0 ||
      max_blocks_per_seq <= 0 || total_query_tokens < 0 ||
      long(total_query_tokens) > long(num_seqs) * max_query_tokens)
    return fail(PA_ERR_INVALID_ARG,
                "invalid sizes: num_seqs=%d total_query_tokens=%d max_query_tokens=%d q_heads=%d "
                "kv_heads=%d max_blocks_per_seq=%d",
                num_seqs, total_query_tokens, max_query_tokens, q_heads, kv_heads,
                max_blocks_per_seq);
  if (q_heads % kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "q_heads (%d) is not a multiple of kv_heads (%d)", q_heads,
                kv_heads);
  const size_t pb = prefill_plan_bytes(num_seqs, max_query_tokens, q_heads, kv_heads);
  if (pb == 0)
    return fail(PA_ERR_UNSUPPORTED, "a prefill plan orders at most %d (sequence, row tile) units",
                pa::kMaxPlanUnits);
  if (!plan || plan_bytes < pb || !aligned(plan, 16))
    return fail(PA_ERR_INVALID_ARG,
                "prefill plan of %zu bytes (16-byte aligned) needed for these sizes, got %zu", pb,
                plan ? plan_bytes : size_t(0));
  if (num_seqs > 0 && (!context_lens || !query_start))
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned(context_lens, 4) || !aligned(query_start, 4))
    return fail(PA_ERR_INVALID_ARG, "misaligned length or offset pointer");
  const int G = q_heads / kv_heads;
  const int per_wg = pa::prefill_rows_per_workgroup();
  pa::PrefillPlanArgs a{context_lens, query_start, static_cast<int32_t*>(plan), num_seqs,
                        int((long(max_query_tokens) * G + per_wg - 1) / per_wg), per_wg, G,
                        total_query_tokens, max_query_tokens, max_blocks_per_seq};
  hipError_t e = pa::launch_prefill_plan(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "plan launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

int pa_prefill_planned(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const float* k_scale, const float* v_scale, const int32_t* block_tables,
                       const int32_t* context_lens, const int32_t* query_start, int num_seqs,
                       int total_query_tokens, int max_query_tokens, int q_heads, int kv_heads,
                       int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                       int max_context_len, float scale, int q_dtype, int kv_dtype,
                       const void* plan, size_t plan_bytes, void* stream) {
  if (!plan) return fail(PA_ERR_INVALID_ARG, "null prefill plan");
  return run_prefill(out, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                     query_start, num_seqs, total_query_tokens, max_query_tokens, q_heads,
                     kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                     max_context_len, scale, q_dtype, kv_dtype, stream, plan, plan_bytes);
}

int pa_verify_varlen(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const float* k_scale, const float* v_scale, const int32_t* block_tables,
                     const int32_t* context_lens, const int32_t* query_start, int num_seqs,
                     int total_query_tokens, int max_query_tokens, int q_heads, int kv_heads,
                     int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                     int max_context_len, float scale, int q_dtype, int kv_dtype,
                     int split_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  Varlen vl;
  vl.query_start = query_start;
  vl.total = total_query_tokens;
  vl.on = true;
  return run_attention(true, out, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                       context_lens, num_seqs, max_query_tokens, q_heads, kv_heads, head_dim,
                       block_size, num_blocks, max_blocks_per_seq, max_context_len, scale,
                       q_dtype, kv_dtype, split_tokens, workspace, workspace_bytes, stream,
                       Append(), vl);
}

}  // extern "C"
