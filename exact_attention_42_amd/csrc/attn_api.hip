// C ABI of libattn.so: argument checks, error reporting, the decode workspace and dispatch
// to the gfx950 kernels. Declarations and the full contract are in include/attn.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>
#include <algorithm>
#include <atomic>

#include "attn.h"
#include "kernels.hpp"

// Fixed device memory for attn_decode_paged_noalloc: the decode's partial results live here
// instead of in an allocated workspace. Each device the library runs on holds its own copy
// until the process ends. On the host `scratch` only names the symbol; its device address is
// taken once per device with hipGetSymbolAddress (scratch_address below) and only that
// address is ever passed to a kernel.
constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local std::string g_last_error;

constexpr int kMaxWorkers = 65536;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return ATTN_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int hip_fail(hipError_t e, const char* where) {
  return fail(ATTN_ERR_HIP, "%s: %s (%d)", where, hipGetErrorString(e), (int)e);
}

int check_scale(float scale) {
  if (!std::isfinite(scale) || scale < 0.f)
    return fail(ATTN_ERR_SCALE, "scale must be finite and >= 0 (got %g)", (double)scale);
  return ATTN_OK;
}

// Returns ATTN_OK and sets *empty when there is nothing to compute.
int check_fwd(const void* q, const void* k, const void* v, void* o, const float* lse, int B,
              int Hq, int Hkv, int Sq, int Sk, int D, float scale, bool* empty) {
  *empty = false;
  if (B < 0 || Sq < 0 || Sk < 0)
    return fail(ATTN_ERR_SHAPE, "B, Sq, Sk must be >= 0 (B=%d Sq=%d Sk=%d)", B, Sq, Sk);
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
    return fail(ATTN_ERR_SHAPE, "need Hq >= 1, Hkv >= 1 and Hq %% Hkv == 0 (Hq=%d Hkv=%d)",
                Hq, Hkv);
  if (D != 64 && D != 128)
    return fail(ATTN_ERR_UNSUPPORTED, "head dimension D=%d not supported (64 or 128)", D);
  if (int rc = check_scale(scale)) return rc;
  if ((long long)B * Hq > 0x7fffffffLL || (long long)Sq > (1 << 30) || (long long)Sk > (1 << 30))
    return fail(ATTN_ERR_SHAPE, "problem too large (B*Hq=%lld, Sq=%d, Sk=%d)",
                (long long)B * Hq, Sq, Sk);
  if (B == 0 || Sq == 0) {
    *empty = true;
    return ATTN_OK;
  }
  if (!q || !o) return fail(ATTN_ERR_NULL, "q and o must not be NULL");
  if (Sk > 0 && (!k || !v)) return fail(ATTN_ERR_NULL, "k and v must not be NULL when Sk > 0");
  if (!aligned(q, 16) || !aligned(o, 16) || !aligned(k, 16) || !aligned(v, 16))
    return fail(ATTN_ERR_ALIGN, "q, k, v and o must be 16-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(ATTN_ERR_ALIGN, "lse must be 4-byte aligned");
  return ATTN_OK;
}

// ---- workspace owned by the library: one buffer per (device, stream), shared by the decode's
// partial results and the split forward's (calls on one stream run in order) ----
//
// Rules:
//  * g_ws_mutex is held from the moment a call takes the library workspace until every kernel
//    of that call is enqueued, so two host threads on one stream can never interleave their
//    kernels over the same buffer;
//  * a buffer that is replaced by a larger one is never freed while the library runs: it goes
//    to g_retired and is freed, with the current ones, only by attn_release_workspace (kernels
//    enqueued earlier may still read it);
//  * the library workspace is refused on a stream that is being captured into a graph: the
//    graph would keep its address while later eager calls replace the buffer. Graphs take a
//    caller workspace through the _ex entry points.
struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mutex;
std::map<std::pair<int, void*>, Workspace> g_ws;
std::vector<std::pair<int, void*>> g_retired;   // (device, buffer) replaced by a larger one

// Compute units of the current device (256 when it cannot be queried).
int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0) {
    (void)hipGetLastError();
    cus = 256;
  }
  return cus;
}

// Worker waves when the caller passes 0: three per CU of the current device, which measured
// fastest (more concurrent block streams only add memory-side contention; fewer leave HBM
// idle). ATTN_DECODE_WORKERS (1..65536) overrides it.
int default_workers() {
  static const int env = [] {
    const char* s = std::getenv("ATTN_DECODE_WORKERS");
    const int x = s ? std::atoi(s) : 0;
    return (x >= 1 && x <= kMaxWorkers) ? x : 0;
  }();
  if (env) return env;
  const int cus = device_cus();
  const int w = 3 * cus;
  return w > kMaxWorkers ? kMaxWorkers : w;
}

// Forced work mapping of the bf16 forward (-1 = chosen per problem). Starts from
// ATTN_FWD_MAPPING = "tile", "pair" or "wide" when set; attn_fwd_force_mapping changes it.
std::atomic<int> g_forced_mapping{-2};   // -2: not read from the environment yet

int forced_fwd_mapping() {
  int m = g_forced_mapping.load(std::memory_order_relaxed);
  if (m != -2) return m;
  const char* s = std::getenv("ATTN_FWD_MAPPING");
  m = -1;
  if (s && std::strcmp(s, "tile") == 0) m = (int)attn::kMapTile;
  if (s && std::strcmp(s, "pair") == 0) m = (int)attn::kMapPair;
  if (s && std::strcmp(s, "wide") == 0) m = (int)attn::kMapWide;
  int expected = -2;
  g_forced_mapping.compare_exchange_strong(expected, m);
  return g_forced_mapping.load(std::memory_order_relaxed);
}

// The library workspace of (current device, stream), at least need bytes. The caller must hold
// g_ws_mutex until its kernels are enqueued.
int get_workspace_locked(void* stream, size_t need, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cap) == hipSuccess &&
      cap != hipStreamCaptureStatusNone)
    return fail(ATTN_ERR_WORKSPACE, "this call needs %zu bytes of workspace on a stream that is "
                "being captured into a graph; the library workspace is never used under "
                "capture: pass a caller workspace through the _ex entry point", need);
  (void)hipGetLastError();
  Workspace& w = g_ws[{dev, stream}];
  if (w.bytes < need) {
    // grow geometrically, so the retired buffers add up to less than the live one
    size_t sz = std::max(need, std::max(w.bytes * 2, (size_t)(1u << 20)));
    void* p = nullptr;
    e = hipMalloc(&p, sz);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(ATTN_ERR_NOMEM, "workspace of %zu bytes: %s", sz, hipGetErrorString(e));
    }
    if (w.ptr) g_retired.push_back({dev, w.ptr});
    w.ptr = p;
    w.bytes = sz;
  }
  *out = w.ptr;
  return ATTN_OK;
}

// Claim block of the wide forward for (current device, stream), at least `words` words: its
// item marks start below any launch mark, and each launch takes a larger mark, so nothing is
// cleared between launches. Launches on one stream run one after another and never share a
// block. None on a stream being captured (a replayed graph would repeat its launch mark) or on
// the per-thread default stream (one handle for many streams): the kernel then runs each item
// on its own workgroup only. The caller holds g_ws_mutex until its kernels are enqueued.
struct ClaimBlock {
  unsigned long long* ptr = nullptr;
  size_t words = 0;
  unsigned long long epoch = 0;
};
std::map<std::pair<int, void*>, ClaimBlock> g_claim;

void claim_block_locked(void* stream, size_t words, unsigned long long** out,
                        unsigned long long* epoch) {
  *out = nullptr;
  if (static_cast<hipStream_t>(stream) == hipStreamPerThread) return;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  int dev = 0;
  if (hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cap) != hipSuccess ||
      cap != hipStreamCaptureStatusNone || hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return;
  }
  ClaimBlock& c = g_claim[{dev, stream}];
  if (c.words < words) {
    const size_t n = std::max(words, std::max(c.words * 2, (size_t)4096));
    void* p = nullptr;
    if (hipMalloc(&p, n * sizeof(unsigned long long)) != hipSuccess) {
      (void)hipGetLastError();
      return;
    }
    if (hipMemsetAsync(p, 0, n * sizeof(unsigned long long),
                       static_cast<hipStream_t>(stream)) != hipSuccess) {
      (void)hipGetLastError();
      (void)hipFree(p);
      return;
    }
    if (c.ptr) g_retired.push_back({dev, c.ptr});
    c.ptr = static_cast<unsigned long long*>(p);
    c.words = n;
  }
  c.epoch += 2;   // even marks for owners; stealers mark with the odd value above
  *out = c.ptr;
  *epoch = c.epoch;
}

// Device address of `scratch` on the current device, looked up once per device (with that
// device current) and kept; a fixed table, so the lookup allocates nothing either.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ATTN_ERR_UNSUPPORTED, "device %d: the fixed scratch supports devices 0..%d", dev,
                kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol,
                      "hipGetSymbolAddress(scratch)");
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

int run_fwd(bool f32, const void* q, const void* k, const void* v, void* o, float* lse, int B,
            int Hq, int Hkv, int Sq, int Sk, int D, int causal, float scale, void* workspace,
            size_t workspace_bytes, void* stream) {
  bool empty;
  if (int rc = check_fwd(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, &empty)) return rc;
  // the bf16 kernel addresses one head's K (and V) through a buffer resource with 32-bit
  // signed offsets
  if (!f32 && (long long)Sk * D * 2 > 0x7fffffffLL)
    return fail(ATTN_ERR_SHAPE, "Sk=%d too long for D=%d: Sk*D*2 must stay below 2^31", Sk, D);
  if (empty) return ok();
  attn::FwdProblem p{q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, causal ? 1 : 0, scale, 1, nullptr,
                     forced_fwd_mapping(), device_cus()};
  std::unique_lock<std::mutex> ws_lock(g_ws_mutex, std::defer_lock);
  if (!f32 && p.mapping < 0) {
    p.nsplit = attn::fwd_bf16_splits(p, p.cus);
    if (p.nsplit > 1) {
      const size_t need = attn::fwd_bf16_workspace_bytes(p, p.nsplit);
      if (workspace) {
        if (workspace_bytes < need)
          return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                      workspace_bytes, need);
        if (!aligned(workspace, 16))
          return fail(ATTN_ERR_WORKSPACE, "workspace must be 16-byte aligned");
        p.workspace = workspace;
      } else {
        ws_lock.lock();
        if (int rc = get_workspace_locked(stream, need, &p.workspace)) return rc;
      }
    }
  }
  if (!f32) {
    // more wide-kernel items than CUs: workgroups that finish early take items of slower XCDs
    const long long items = attn::fwd_wide_items(p);
    if (items > p.cus) {
      if (!ws_lock.owns_lock()) ws_lock.lock();
      claim_block_locked(stream, attn::wide_claim_words(items), &p.claim, &p.epoch);
    }
  }
  hipError_t e = f32 ? attn::launch_fwd_f32(p, static_cast<hipStream_t>(stream))
                     : attn::launch_fwd_bf16(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, f32 ? "attn_fwd_f32 launch" : "attn_fwd launch");
  return ok();
}

int run_fwd_paged(const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_table, const int32_t* cu_seqlens_q,
                  const int32_t* ctx_lens, void* o, float* lse, int B, int T, int Hq, int Hkv,
                  int D, int block_size, int max_q, int max_ctx, int table_stride,
                  int num_blocks, int causal, float scale, void* workspace,
                  size_t workspace_bytes, void* stream) {
  if (B < 0 || T < 0 || max_q < 0 || max_ctx < 0)
    return fail(ATTN_ERR_SHAPE, "B, T, max_q and max_ctx must be >= 0 (B=%d T=%d max_q=%d "
                "max_ctx=%d)", B, T, max_q, max_ctx);
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
    return fail(ATTN_ERR_SHAPE, "need Hq >= 1, Hkv >= 1 and Hq %% Hkv == 0 (Hq=%d Hkv=%d)",
                Hq, Hkv);
  if (table_stride < 1)
    return fail(ATTN_ERR_SHAPE, "table_stride must be >= 1 (got %d)", table_stride);
  if ((long long)B * Hq > 0x7fffffffLL || (long long)T * Hq > 0x7fffffffLL ||
      max_q > (1 << 30) || max_ctx > (1 << 30) || (long long)B * table_stride > 0x7fffffffLL)
    return fail(ATTN_ERR_SHAPE, "problem too large (B*Hq=%lld T*Hq=%lld max_q=%d max_ctx=%d)",
                (long long)B * Hq, (long long)T * Hq, max_q, max_ctx);
  if (D != 64 && D != 128)
    return fail(ATTN_ERR_UNSUPPORTED, "head dimension D=%d not supported (64 or 128)", D);
  if (block_size != 16)
    return fail(ATTN_ERR_UNSUPPORTED, "block_size=%d not supported (16)", block_size);
  if (int rc = check_scale(scale)) return rc;
  if (B == 0 || T == 0 || max_q == 0) return ok();
  if (!q || !k_cache || !v_cache || !block_table || !cu_seqlens_q || !ctx_lens || !o)
    return fail(ATTN_ERR_NULL, "q, k_cache, v_cache, block_table, cu_seqlens_q, ctx_lens and o "
                "must not be NULL");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16))
    return fail(ATTN_ERR_ALIGN, "q, k_cache, v_cache and o must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(cu_seqlens_q, 4) || !aligned(ctx_lens, 4) ||
      (lse && !aligned(lse, 4)))
    return fail(ATTN_ERR_ALIGN, "block_table, cu_seqlens_q, ctx_lens and lse must be 4-byte "
                "aligned");
  attn::PagedProblem p{};
  p.q = q; p.k_cache = k_cache; p.v_cache = v_cache; p.block_table = block_table;
  p.cu_seqlens_q = cu_seqlens_q; p.ctx_lens = ctx_lens; p.o = o; p.lse = lse;
  p.B = B; p.T = T; p.Hq = Hq; p.Hkv = Hkv; p.D = D; p.max_q = max_q; p.max_ctx = max_ctx;
  p.table_stride = table_stride; p.num_blocks = num_blocks; p.causal = causal ? 1 : 0;
  p.scale = scale;
  p.nsplit = attn::fwd_paged_splits(p, device_cus());
  p.workspace = nullptr;
  std::unique_lock<std::mutex> ws_lock(g_ws_mutex, std::defer_lock);
  if (p.nsplit > 1) {
    const size_t need = attn::fwd_paged_workspace_bytes(p, p.nsplit);
    if (workspace) {
      if (workspace_bytes < need)
        return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                    workspace_bytes, need);
      if (!aligned(workspace, 16))
        return fail(ATTN_ERR_WORKSPACE, "workspace must be 16-byte aligned");
      p.workspace = workspace;
    } else {
      ws_lock.lock();
      if (int rc = get_workspace_locked(stream, need, &p.workspace)) return rc;
    }
  }
  hipError_t e = attn::launch_fwd_paged(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "attn_fwd_paged launch");
  return ok();
}

int run_decode(const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_table, const int32_t* ctx_lens, void* o, float* lse, int B,
               int Hq, int Hkv, int D, int block_size, float scale, int table_stride,
               int num_blocks, int num_workers, void* workspace, size_t workspace_bytes,
               void* stream, bool use_scratch = false) {
  if (B < 0) return fail(ATTN_ERR_SHAPE, "B must be >= 0 (B=%d)", B);
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
    return fail(ATTN_ERR_SHAPE, "need Hq >= 1, Hkv >= 1 and Hq %% Hkv == 0 (Hq=%d Hkv=%d)",
                Hq, Hkv);
  if (B > 65535 || Hkv > 65535)
    return fail(ATTN_ERR_SHAPE, "B and Hkv must be <= 65535 (B=%d Hkv=%d)", B, Hkv);
  if (Hq / Hkv > 16)
    return fail(ATTN_ERR_UNSUPPORTED, "decode supports Hq/Hkv <= 16 (got %d)", Hq / Hkv);
  if (D != 64 && D != 128)
    return fail(ATTN_ERR_UNSUPPORTED, "head dimension D=%d not supported (64 or 128)", D);
  if (block_size != 16)
    return fail(ATTN_ERR_UNSUPPORTED, "block_size=%d not supported (16)", block_size);
  if (int rc = check_scale(scale)) return rc;
  if (num_workers < 0 || num_workers > kMaxWorkers)
    return fail(ATTN_ERR_SHAPE, "num_workers must be in 0..%d (got %d)", kMaxWorkers, num_workers);
  if (B == 0) return ok();
  if (!q || !k_cache || !v_cache || !block_table || !ctx_lens || !o)
    return fail(ATTN_ERR_NULL, "q, k_cache, v_cache, block_table, ctx_lens and o must not be NULL");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16))
    return fail(ATTN_ERR_ALIGN, "q, k_cache, v_cache and o must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(ctx_lens, 4) || (lse && !aligned(lse, 4)))
    return fail(ATTN_ERR_ALIGN, "block_table, ctx_lens and lse must be 4-byte aligned");
  const int workers = num_workers ? num_workers : default_workers();
  const size_t need = attn::decode_workspace_bytes(B, Hkv, Hq / Hkv, D, workers);
  void* ws = workspace;
  std::unique_lock<std::mutex> ws_lock(g_ws_mutex, std::defer_lock);
  if (use_scratch) {
    // the fixed device array: nothing is allocated; a problem that does not fit is refused
    if (need > kScratchBytes)
      return fail(ATTN_ERR_WORKSPACE, "this decode needs %zu bytes of partial results, more than "
                  "the %zu bytes of fixed scratch of attn_decode_paged_noalloc (fewer worker "
                  "waves, a smaller batch, or attn_decode_paged_ex with a caller workspace)",
                  need, kScratchBytes);
    if (int rc = scratch_address(&ws)) return rc;
  } else if (ws) {
    if (workspace_bytes < need)
      return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                  workspace_bytes, need);
    if (!aligned(ws, 16)) return fail(ATTN_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  } else {
    ws_lock.lock();
    if (int rc = get_workspace_locked(stream, need, &ws)) return rc;
  }
  attn::DecodeProblem p;
  p.q = q; p.k_cache = k_cache; p.v_cache = v_cache;
  p.block_table = block_table; p.ctx_lens = ctx_lens; p.o = o; p.lse = lse;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.D = D; p.block_size = block_size;
  p.table_stride = table_stride; p.num_blocks = num_blocks; p.workers = workers;
  p.scale = scale;
  p.workspace = ws;
  hipError_t e = attn::launch_decode_paged(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "attn_decode_paged launch");
  return ok();
}

int run_add_rms_norm(const void* x, const void* residual, const void* weight, void* out,
                     void* residual_out, int M, int d, float eps, void* stream) {
  if (M < 0 || d < 0) return fail(ATTN_ERR_SHAPE, "M and d must be >= 0 (M=%d d=%d)", M, d);
  if (d == 0 || d % 8 != 0 || d > 65536)
    return fail(ATTN_ERR_UNSUPPORTED, "row length d=%d not supported (a multiple of 8, 8..65536)",
                d);
  if (!std::isfinite(eps) || eps < 0.f)
    return fail(ATTN_ERR_SCALE, "eps must be finite and >= 0 (got %g)", (double)eps);
  if (M == 0) return ok();
  if (!x || !residual || !weight || !out || !residual_out)
    return fail(ATTN_ERR_NULL, "x, residual, weight, out and residual_out must not be NULL");
  if (!aligned(x, 16) || !aligned(residual, 16) || !aligned(weight, 16) || !aligned(out, 16) ||
      !aligned(residual_out, 16))
    return fail(ATTN_ERR_ALIGN, "x, residual, weight, out and residual_out must be 16-byte aligned");
  attn::NormProblem p{x, residual, weight, out, residual_out, M, d, eps};
  hipError_t e = attn::launch_add_rms_norm(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "attn_add_rms_norm launch");
  return ok();
}

int run_rope_cache_write(const void* q, const void* k, const void* v, void* q_out,
                         void* k_cache, void* v_cache, const int32_t* block_table,
                         const int32_t* positions, const int32_t* seq_ids, int T, int num_seqs,
                         int Hq, int Hkv, int D, int block_size, int table_stride,
                         int num_blocks, float base, void* stream) {
  if (T < 0 || num_seqs < 0)
    return fail(ATTN_ERR_SHAPE, "T and num_seqs must be >= 0 (T=%d num_seqs=%d)", T, num_seqs);
  if (Hq < 1 || Hkv < 1 || table_stride < 1)
    return fail(ATTN_ERR_SHAPE, "need Hq >= 1, Hkv >= 1 and table_stride >= 1 (Hq=%d Hkv=%d "
                "table_stride=%d)", Hq, Hkv, table_stride);
  if (!seq_ids && T > num_seqs)
    return fail(ATTN_ERR_SHAPE, "without seq_ids token t is sequence t, so T=%d must be <= "
                "num_seqs=%d", T, num_seqs);
  if (D != 64 && D != 128)
    return fail(ATTN_ERR_UNSUPPORTED, "head dimension D=%d not supported (64 or 128)", D);
  if (block_size != 16)
    return fail(ATTN_ERR_UNSUPPORTED, "block_size=%d not supported (16)", block_size);
  if (!std::isfinite(base) || !(base > 0.f))
    return fail(ATTN_ERR_SCALE, "rope base must be finite and > 0 (got %g)", (double)base);
  if (T == 0) return ok();
  if (!q || !k || !v || !q_out || !k_cache || !v_cache || !block_table || !positions)
    return fail(ATTN_ERR_NULL, "q, k, v, q_out, k_cache, v_cache, block_table and positions "
                "must not be NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(q_out, 16) ||
      !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(ATTN_ERR_ALIGN, "q, k, v, q_out, k_cache and v_cache must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(positions, 4) || (seq_ids && !aligned(seq_ids, 4)))
    return fail(ATTN_ERR_ALIGN, "block_table, positions and seq_ids must be 4-byte aligned");
  attn::RopeProblem p{q, k, v, q_out, k_cache, v_cache, block_table, positions, seq_ids,
                      T, num_seqs, Hq, Hkv, D, table_stride, num_blocks, base};
  hipError_t e = attn::launch_rope_cache_write(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "attn_rope_cache_write launch");
  return ok();
}

}  // namespace

extern "C" {

int attn_rope_cache_write(const void* q, const void* k, const void* v, void* q_out,
                          void* k_cache, void* v_cache, const int32_t* block_table,
                          const int32_t* positions, const int32_t* seq_ids, int T,
                          int num_seqs, int Hq, int Hkv, int D, int block_size,
                          int table_stride, int num_blocks, float base, hipStream_t stream) {
  return run_rope_cache_write(q, k, v, q_out, k_cache, v_cache, block_table, positions,
                              seq_ids, T, num_seqs, Hq, Hkv, D, block_size, table_stride,
                              num_blocks, base, stream);
}

int attn_add_rms_norm(const void* x, const void* residual, const void* weight, void* out,
                      void* residual_out, int M, int d, float eps, hipStream_t stream) {
  return run_add_rms_norm(x, residual, weight, out, residual_out, M, d, eps, stream);
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
             int Hkv, int Sq, int Sk, int D, int causal, float scale, hipStream_t stream) {
  return run_fwd(false, q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, causal, scale, nullptr, 0,
                 stream);
}

int attn_fwd_force_mapping(int mapping) {
  const int prev = forced_fwd_mapping();
  const int m = (mapping >= (int)attn::kMapTile && mapping <= (int)attn::kMapWide) ? mapping : -1;
  g_forced_mapping.store(m, std::memory_order_relaxed);
  return prev;
}

int attn_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                 int Hq, int Hkv, int Sq, int Sk, int D, int causal, float scale, hipStream_t stream) {
  return run_fwd(true, q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, causal, scale, nullptr, 0,
                 stream);
}

int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                int Hkv, int Sq, int Sk, int D, int causal, float scale, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
  return run_fwd(false, q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, causal, scale, workspace,
                 workspace_bytes, stream);
}

size_t attn_fwd_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal) {
  if (B < 0 || Sq < 0 || Sk < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || (D != 64 && D != 128) ||
      (long long)B * Hq > 0x7fffffffLL || Sq > (1 << 30) || Sk > (1 << 30))
    return 0;
  attn::FwdProblem p{nullptr, nullptr, nullptr, nullptr, nullptr, B, Hq, Hkv, Sq, Sk, D,
                     causal ? 1 : 0, 1.0f, 1, nullptr, forced_fwd_mapping(), device_cus()};
  if (p.mapping >= 0) return 0;
  return attn::fwd_bf16_workspace_bytes(p, attn::fwd_bf16_splits(p, device_cus()));
}

int attn_fwd_paged(const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* block_table, const int32_t* cu_seqlens_q,
                   const int32_t* ctx_lens, void* o, float* lse, int B, int T, int Hq, int Hkv,
                   int D, int block_size, int max_q, int max_ctx, int table_stride,
                   int num_blocks, int causal, float scale, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  return run_fwd_paged(q, k_cache, v_cache, block_table, cu_seqlens_q, ctx_lens, o, lse, B, T,
                       Hq, Hkv, D, block_size, max_q, max_ctx, table_stride, num_blocks, causal,
                       scale, workspace, workspace_bytes, stream);
}

size_t attn_fwd_paged_workspace_bytes(int B, int T, int Hq, int Hkv, int D, int max_q,
                                      int max_ctx, int causal) {
  if (B < 0 || T < 0 || max_q < 0 || max_ctx < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 ||
      (D != 64 && D != 128) || (long long)B * Hq > 0x7fffffffLL ||
      (long long)T * Hq > 0x7fffffffLL || max_q > (1 << 30) || max_ctx > (1 << 30))
    return 0;
  attn::PagedProblem p{};
  p.B = B; p.T = T; p.Hq = Hq; p.Hkv = Hkv; p.D = D; p.max_q = max_q; p.max_ctx = max_ctx;
  p.causal = causal ? 1 : 0;
  return attn::fwd_paged_workspace_bytes(p, attn::fwd_paged_splits(p, device_cus()));
}

int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, const int32_t* ctx_lens, void* o, int B,
                      int Hq, int Hkv, int D, int block_size, float scale, hipStream_t stream) {
  return run_decode(q, k_cache, v_cache, block_table, ctx_lens, o, nullptr, B, Hq, Hkv, D,
                    block_size, scale, 0, 0, 0, nullptr, 0, stream);
}

int attn_decode_paged_full(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_table, const int32_t* ctx_lens, void* o,
                           float* lse, int B, int Hq, int Hkv, int D, int block_size,
                           float scale, int table_stride, int num_blocks, int num_workers,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return run_decode(q, k_cache, v_cache, block_table, ctx_lens, o, lse, B, Hq, Hkv, D,
                    block_size, scale, table_stride, num_blocks, num_workers, workspace,
                    workspace_bytes, stream);
}

int attn_decode_paged_ex(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_table, const int32_t* ctx_lens, void* o, int B,
                         int Hq, int Hkv, int D, int block_size, float scale,
                         int block_table_stride, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  return run_decode(q, k_cache, v_cache, block_table, ctx_lens, o, nullptr, B, Hq, Hkv, D,
                    block_size, scale, block_table_stride, 0, 0, workspace, workspace_bytes,
                    stream);
}

int attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* ctx_lens, void* o,
                              float* lse, int B, int Hq, int Hkv, int D, int block_size,
                              float scale, int table_stride, int num_blocks, int num_workers,
                              hipStream_t stream) {
  return run_decode(q, k_cache, v_cache, block_table, ctx_lens, o, lse, B, Hq, Hkv, D,
                    block_size, scale, table_stride, num_blocks, num_workers, nullptr, 0, stream,
                    /*use_scratch=*/true);
}

size_t attn_decode_noalloc_max_bytes(void) { return kScratchBytes; }

size_t attn_decode_workspace_bytes_ex(int B, int Hq, int Hkv, int D, int num_workers) {
  if (B < 0 || B > 65535 || Hq < 1 || Hkv < 1 || Hkv > 65535 || Hq % Hkv != 0 ||
      Hq / Hkv > 16 || (D != 64 && D != 128) || num_workers < 0 || num_workers > kMaxWorkers)
    return 0;
  return attn::decode_workspace_bytes(B, Hkv, Hq / Hkv, D,
                                      num_workers ? num_workers : default_workers());
}

size_t attn_decode_workspace_bytes(int B, int Hq, int D) {
  // the largest need over every Hkv the decode accepts for Hq (Hkv divides Hq, Hq / Hkv <= 16)
  size_t best = 0;
  for (int hkv = 1; hkv <= Hq && hkv <= 65535; ++hkv) {
    if (Hq % hkv != 0 || Hq / hkv > 16) continue;
    best = std::max(best, attn_decode_workspace_bytes_ex(B, Hq, hkv, D, 0));
  }
  return best;
}

int attn_decode_default_workers(void) { return default_workers(); }

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "null pointer";
    case ATTN_ERR_SHAPE: return "invalid shape";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_ALIGN: return "misaligned pointer";
    case ATTN_ERR_SCALE: return "invalid scale";
    case ATTN_ERR_HIP: return "HIP runtime error";
    case ATTN_ERR_NOMEM: return "out of device memory";
    case ATTN_ERR_WORKSPACE: return "invalid workspace";
    default: return "unknown status";
  }
}

const char* attn_last_error(void) { return g_last_error.c_str(); }

void attn_release_workspace(void) {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  int cur = 0;
  bool have_cur = hipGetDevice(&cur) == hipSuccess;
  for (auto& kv : g_ws) {
    if (kv.second.ptr) {
      if (hipSetDevice(kv.first.first) == hipSuccess) (void)hipFree(kv.second.ptr);
    }
  }
  for (auto& kv : g_claim) {
    if (kv.second.ptr) {
      if (hipSetDevice(kv.first.first) == hipSuccess) (void)hipFree(kv.second.ptr);
    }
  }
  for (auto& r : g_retired) {
    if (hipSetDevice(r.first) == hipSuccess) (void)hipFree(r.second);
  }
  g_ws.clear();
  g_claim.clear();
  g_retired.clear();
  if (have_cur) (void)hipSetDevice(cur);
}

int attn_abi_version(void) { return 10; }

}  // extern "C"
