// xq_api.cpp — the C ABI declared in include/xq.h.
//
// Every entry point checks its arguments on the host (null pointers, shapes,
// alignment, then the device) before any launch, and answers a refusal with
// a status plus a thread-local sentence naming the gate ("25 — Writing XPU
// Kernels", section 25.6: a refusal names the gate that refused; section 25.5:
// a base short of the alignment the loads need is refused by name). Nothing
// falls back to another kernel or to the host.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/xq.h"
#include "xq_launch.h"

namespace {

thread_local char g_err[256] = "";

xq_status fail(xq_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

xq_status ok() {
  g_err[0] = '\0';
  return XQ_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int kMaxDevices = 64;
// 0 = not checked, 1 = gfx950, 2 = other architecture.
std::atomic<int> g_dev_state[kMaxDevices];

xq_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(XQ_E_DEVICE, "no current HIP device");
  if (dev >= kMaxDevices) return fail(XQ_E_DEVICE, "device %d beyond the library's table", dev);
  int st = g_dev_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
      return fail(XQ_E_DEVICE, "hipGetDeviceProperties failed on device %d", dev);
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev_state[dev].store(st, std::memory_order_release);
  }
  if (st != 1) return fail(XQ_E_DEVICE, "device %d is not gfx950", dev);
  return XQ_OK;
}

xq_status check_k(int64_t K, int64_t kmax) {
  if (K < 256 || K % 256 != 0) return fail(XQ_E_SHAPE, "K=%lld not a positive multiple of 256", (long long)K);
  if (kmax > 0 && K > kmax)
    return fail(XQ_E_SHAPE, "K=%lld above the largest supported K=%lld", (long long)K, (long long)kmax);
  return XQ_OK;
}

constexpr int64_t kMaxInt = 2147483647LL;
// Row counts stay below 2^30 so that no 32-bit row index in a kernel can wrap.
constexpr int64_t kMaxRows = 1LL << 30;
constexpr int64_t kIdMaxPairs = 1LL << 20;  // (token, slot) pairs of one grouped product
constexpr int64_t kIdMaxExperts = 1024;

// A call that needs `need` bytes of caller workspace: a null or short
// workspace is refused by name (shape stage), a misaligned one at the
// alignment stage (check_workspace_align).
xq_status check_workspace(const void* ws, size_t ws_bytes, size_t need, const char* query) {
  if (need == 0) return XQ_OK;
  if (!ws)
    return fail(XQ_E_NULL, "workspace is NULL; this call needs %zu bytes (%s)", need, query);
  if (ws_bytes < need)
    return fail(XQ_E_SHAPE, "workspace_bytes=%zu below the %zu bytes this call needs (%s)",
                ws_bytes, need, query);
  return XQ_OK;
}

xq_status check_workspace_align(const void* ws, size_t need) {
  if (need > 0 && !aligned(ws, 256)) return fail(XQ_E_ALIGN, "workspace not 256-byte aligned");
  return XQ_OK;
}

xq_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(XQ_E_LAUNCH, "%s launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

xq_status xq_quantize_q8k(void* xq, const float* x, int64_t rows, int64_t K, void* stream) {
  if (!xq) return fail(XQ_E_NULL, "xq is NULL");
  if (!x) return fail(XQ_E_NULL, "x is NULL");
  if (rows < 1) return fail(XQ_E_SHAPE, "rows=%lld below 1", (long long)rows);
  if (xq_status s = check_k(K, 0)) return s;
  if (rows > kMaxInt / (K / 256))
    return fail(XQ_E_SHAPE, "rows*K/256 = %lld*%lld exceeds 2^31-1 blocks", (long long)rows,
                (long long)(K / 256));
  if (!aligned(xq, 16)) return fail(XQ_E_ALIGN, "xq not 16-byte aligned");
  if (!aligned(x, 4)) return fail(XQ_E_ALIGN, "x not 4-byte aligned");
  if (xq_status s = check_device()) return s;
  return launched(xq::launch_quantize_q8k(xq, x, rows, K, static_cast<hipStream_t>(stream)),
                  "xq_quantize_q8k");
}

xq_status xq_gemv_q4k(float* y, const void* w, const void* xq, int64_t N, int64_t K,
                      void* stream) {
  if (!y) return fail(XQ_E_NULL, "y is NULL");
  if (!w) return fail(XQ_E_NULL, "w is NULL");
  if (!xq) return fail(XQ_E_NULL, "xq is NULL");
  if (N < 1 || N > kMaxRows) return fail(XQ_E_SHAPE, "N=%lld outside 1..2^30", (long long)N);
  if (xq_status s = check_k(K, XQ_MAX_K)) return s;
  if (!aligned(y, 4)) return fail(XQ_E_ALIGN, "y not 4-byte aligned");
  if (!aligned(w, 16)) return fail(XQ_E_ALIGN, "w not 16-byte aligned");
  if (!aligned(xq, 16)) return fail(XQ_E_ALIGN, "xq not 16-byte aligned");
  if (xq_status s = check_device()) return s;
  return launched(xq::launch_gemv_q4k(y, w, xq, N, K, static_cast<hipStream_t>(stream)),
                  "xq_gemv_q4k");
}

xq_status xq_gemv_q4k_q8k(float* y, void* yq, const void* w, const void* xq, int64_t N,
                          int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  if (!y) return fail(XQ_E_NULL, "y is NULL");
  if (!yq) return fail(XQ_E_NULL, "yq is NULL");
  if (!w) return fail(XQ_E_NULL, "w is NULL");
  if (!xq) return fail(XQ_E_NULL, "xq is NULL");
  if (N < 256 || N % 256 != 0 || N > (1LL << 22))
    return fail(XQ_E_SHAPE, "N=%lld not a multiple of 256 in 256..2^22", (long long)N);
  if (xq_status s = check_k(K, XQ_MAX_K)) return s;
  const size_t need = xq::gemv_q4k_q8k_workspace_bytes(N);
  if (xq_status s = check_workspace(workspace, workspace_bytes, need,
                                    "xq_gemv_q4k_q8k_workspace_bytes"))
    return s;
  if (!aligned(y, 4)) return fail(XQ_E_ALIGN, "y not 4-byte aligned");
  if (!aligned(yq, 16)) return fail(XQ_E_ALIGN, "yq not 16-byte aligned");
  if (!aligned(w, 16)) return fail(XQ_E_ALIGN, "w not 16-byte aligned");
  if (!aligned(xq, 16)) return fail(XQ_E_ALIGN, "xq not 16-byte aligned");
  if (xq_status s = check_workspace_align(workspace, need)) return s;
  if (xq_status s = check_device()) return s;
  return launched(xq::launch_gemv_q4k_q8k(y, yq, w, xq, N, K, workspace, workspace_bytes,
                                          static_cast<hipStream_t>(stream)),
                  "xq_gemv_q4k_q8k");
}

size_t xq_gemv_q4k_q8k_workspace_bytes(int64_t N) { return xq::gemv_q4k_q8k_workspace_bytes(N); }

xq_status xq_gemv_iq4nl(float* y, const void* w, const void* xq, int64_t N, int64_t K,
                        void* stream) {
  if (!y) return fail(XQ_E_NULL, "y is NULL");
  if (!w) return fail(XQ_E_NULL, "w is NULL");
  if (!xq) return fail(XQ_E_NULL, "xq is NULL");
  if (N < 1 || N > kMaxRows) return fail(XQ_E_SHAPE, "N=%lld outside 1..2^30", (long long)N);
  if (xq_status s = check_k(K, XQ_MAX_K)) return s;
  if (!aligned(y, 4)) return fail(XQ_E_ALIGN, "y not 4-byte aligned");
  if (!aligned(w, 16)) return fail(XQ_E_ALIGN, "w not 16-byte aligned");
  if (!aligned(xq, 16)) return fail(XQ_E_ALIGN, "xq not 16-byte aligned");
  if (xq_status s = check_device()) return s;
  return launched(xq::launch_gemv_iq4nl(y, w, xq, N, K, static_cast<hipStream_t>(stream)),
                  "xq_gemv_iq4nl");
}

xq_status xq_gemv_q4_0(float* y, const void* w, const void* xq, int64_t N, int64_t K,
                       void* stream) {
  if (!y) return fail(XQ_E_NULL, "y is NULL");
  if (!w) return fail(XQ_E_NULL, "w is NULL");
  if (!xq) return fail(XQ_E_NULL, "xq is NULL");
  if (N < 1 || N > kMaxRows) return fail(XQ_E_SHAPE, "N=%lld outside 1..2^30", (long long)N);
  if (xq_status s = check_k(K, XQ_MAX_K)) return s;
  if (!aligned(y, 4)) return fail(XQ_E_ALIGN, "y not 4-byte aligned");
  if (!aligned(w, 16)) return fail(XQ_E_ALIGN, "w not 16-byte aligned");
  if (!aligned(xq, 16)) return fail(XQ_E_ALIGN, "xq not 16-byte aligned");
  if (xq_status s = check_device()) return s;
  return launched(xq::launch_gemv_q4_0(y, w, xq, N, K, static_cast<hipStream_t>(stream)),
                  "xq_gemv_q4_0");
}

static xq_status check_id(float* y, const void* slab, const void* xq,
                   const int32_t* sel, int64_t n_experts, int64_t used, int64_t rows, int64_t K,
                   int64_t x_stride_blocks) {
  if (!y) return fail(XQ_E_NULL, "y is NULL");
  if (!slab) return fail(XQ_E_NULL, "slab is NULL");
  if (!xq) return fail(XQ_E_NULL, "xq is NULL");
  if (!sel) return fail(XQ_E_NULL, "sel is NULL");
  if (n_experts < 1) return fail(XQ_E_SHAPE, "n_experts=%lld below 1", (long long)n_experts);
  if (used < 1 || used > 65535)
    return fail(XQ_E_SHAPE, "used=%lld outside 1..65535", (long long)used);
  if (rows < 1 || rows > kMaxRows)
    return fail(XQ_E_SHAPE, "rows=%lld outside 1..2^30", (long long)rows);
  if (n_experts > kMaxRows / rows)
    return fail(XQ_E_SHAPE, "n_experts*rows = %lld*%lld above 2^30", (long long)n_experts,
                (long long)rows);
  if (xq_status s = check_k(K, XQ_MAX_K)) return s;
  if (x_stride_blocks != 0 && x_stride_blocks != K / 256)
    return fail(XQ_E_SHAPE, "x_stride_blocks=%lld is neither 0 nor K/256=%lld",
                (long long)x_stride_blocks, (long long)(K / 256));
  if (!aligned(y, 4)) return fail(XQ_E_ALIGN, "y not 4-byte aligned");
  if (!aligned(slab, 16)) return fail(XQ_E_ALIGN, "slab not 16-byte aligned");
  if (!aligned(xq, 16)) return fail(XQ_E_ALIGN, "xq not 16-byte aligned");
  if (!aligned(sel, 4)) return fail(XQ_E_ALIGN, "sel not 4-byte aligned");
  return check_device();
}

xq_status xq_gemv_q4k_id(float* y, const void* slab, const void* xq, const int32_t* sel,
                         int64_t n_experts, int64_t used, int64_t rows, int64_t K,
                         int64_t x_stride_blocks, void* stream) {
  if (xq_status s = check_id(y, slab, xq, sel, n_experts, used, rows, K,
                             x_stride_blocks))
    return s;
  return launched(xq::launch_gemv_q4k_id(y, slab, xq, sel, n_experts, used, rows, K,
                                         x_stride_blocks, static_cast<hipStream_t>(stream)),
                  "xq_gemv_q4k_id");
}

xq_status xq_gemv_iq4nl_id(float* y, const void* slab, const void* xq, const int32_t* sel,
                           int64_t n_experts, int64_t used, int64_t rows, int64_t K,
                           int64_t x_stride_blocks, void* stream) {
  if (xq_status s = check_id(y, slab, xq, sel, n_experts, used, rows, K,
                             x_stride_blocks))
    return s;
  return launched(xq::launch_gemv_iq4nl_id(y, slab, xq, sel, n_experts, used, rows, K,
                                           x_stride_blocks, static_cast<hipStream_t>(stream)),
                  "xq_gemv_iq4nl_id");
}

// The small-M product's gates up to the workspace: null pointers, shape.
static xq_status check_gemm(const float* y, const void* w, const void* xq, int64_t M, int64_t N,
                            int64_t K) {
  if (!y) return fail(XQ_E_NULL, "y is NULL");
  if (!w) return fail(XQ_E_NULL, "w is NULL");
  if (!xq) return fail(XQ_E_NULL, "xq is NULL");
  if (M < 1 || M > kMaxRows) return fail(XQ_E_SHAPE, "M=%lld outside 1..2^30", (long long)M);
  if (N < 1 || N > kMaxRows) return fail(XQ_E_SHAPE, "N=%lld outside 1..2^30", (long long)N);
  if (xq_status s = check_k(K, 0)) return s;
  if (K / 256 > kMaxInt) return fail(XQ_E_SHAPE, "K=%lld too large", (long long)K);
  if (((M + 63) / 64) * ((N + 127) / 128) > kMaxInt)
    return fail(XQ_E_SHAPE, "M*N too large for one launch");
  // The kernel addresses its inputs with 32-bit byte offsets. (Compared by
  // division: a row's bytes fit in int64, a matrix's need not.)
  const int64_t nb = K / 256;
  if (M > ((1LL << 31) - 1) / (nb * 320))
    return fail(XQ_E_SHAPE, "xq of M=%lld rows reaches 2 GiB", (long long)M);
  if (N > ((1LL << 31) - 1) / (nb * 144))
    return fail(XQ_E_SHAPE, "w of N=%lld rows reaches 2 GiB", (long long)N);
  return XQ_OK;
}

static xq_status check_gemm_align(const float* y, const void* w, const void* xq) {
  if (!aligned(y, 4)) return fail(XQ_E_ALIGN, "y not 4-byte aligned");
  if (!aligned(w, 16)) return fail(XQ_E_ALIGN, "w not 16-byte aligned");
  if (!aligned(xq, 16)) return fail(XQ_E_ALIGN, "xq not 16-byte aligned");
  return XQ_OK;
}

xq_status xq_gemm_q4k_small_m(float* y, const void* w, const void* xq, int64_t M, int64_t N,
                              int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  if (xq_status s = check_gemm(y, w, xq, M, N, K)) return s;
  const size_t need = xq::gemm_q4k_workspace_bytes(M, N, K);
  if (xq_status s = check_workspace(workspace, workspace_bytes, need,
                                    "xq_gemm_q4k_small_m_workspace_bytes"))
    return s;
  if (xq_status s = check_gemm_align(y, w, xq)) return s;
  if (xq_status s = check_workspace_align(workspace, need)) return s;
  if (xq_status s = check_device()) return s;
  return launched(xq::launch_gemm_q4k(y, w, xq, M, N, K, workspace, workspace_bytes,
                                      static_cast<hipStream_t>(stream)),
                  "xq_gemm_q4k_small_m");
}

xq_status xq_gemm_q4k_small_m_noalloc(float* y, const void* w, const void* xq, int64_t M,
                                      int64_t N, int64_t K, void* stream) {
  if (xq_status s = check_gemm(y, w, xq, M, N, K)) return s;
  const size_t need = xq::gemm_q4k_workspace_bytes(M, N, K);
  if (need > xq::gemm_q4k_noalloc_scratch_bytes())
    return fail(XQ_E_SHAPE,
                "M=%lld N=%lld K=%lld needs %zu bytes of split-K scratch, above the %zu bytes "
                "xq_gemm_q4k_small_m_noalloc holds (xq_gemm_q4k_small_m with a caller workspace "
                "takes any shape)",
                (long long)M, (long long)N, (long long)K, need,
                xq::gemm_q4k_noalloc_scratch_bytes());
  if (xq_status s = check_gemm_align(y, w, xq)) return s;
  if (xq_status s = check_device()) return s;
  return launched(xq::launch_gemm_q4k_noalloc(y, w, xq, M, N, K, static_cast<hipStream_t>(stream)),
                  "xq_gemm_q4k_small_m_noalloc");
}

size_t xq_gemm_q4k_small_m_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  return xq::gemm_q4k_workspace_bytes(M, N, K);
}

xq_status xq_gemm_q4k_id(float* y, const void* slab, const void* xq, const int32_t* ids,
                         int64_t n_tokens, int64_t n_used, int64_t n_experts, int64_t rows,
                         int64_t K, int64_t x_per_slot, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (!y) return fail(XQ_E_NULL, "y is NULL");
  if (!slab) return fail(XQ_E_NULL, "slab is NULL");
  if (!xq) return fail(XQ_E_NULL, "xq is NULL");
  if (!ids) return fail(XQ_E_NULL, "ids is NULL");
  if (n_used < 1 || n_used > kIdMaxPairs)
    return fail(XQ_E_SHAPE, "n_used=%lld outside 1..2^20", (long long)n_used);
  if (n_tokens < 1 || n_tokens > kIdMaxPairs / n_used)
    return fail(XQ_E_SHAPE, "n_tokens*n_used = %lld*%lld outside 1..2^20", (long long)n_tokens,
                (long long)n_used);
  if (n_experts < 1 || n_experts > kIdMaxExperts)
    return fail(XQ_E_SHAPE, "n_experts=%lld outside 1..1024", (long long)n_experts);
  if (rows < 1 || rows > kMaxRows)
    return fail(XQ_E_SHAPE, "rows=%lld outside 1..2^30", (long long)rows);
  if (xq_status s = check_k(K, 0)) return s;
  if (K / 256 > kMaxInt) return fail(XQ_E_SHAPE, "K=%lld too large", (long long)K);
  if (x_per_slot != 0 && x_per_slot != 1)
    return fail(XQ_E_SHAPE, "x_per_slot=%lld is neither 0 nor 1", (long long)x_per_slot);
  const int64_t n_pairs = n_tokens * n_used;
  const int64_t xrows = x_per_slot ? n_pairs : n_tokens;
  // The kernel addresses one expert's weights and all of xq with 32-bit byte
  // offsets (compared by division, as in the dense product).
  if (rows > ((1LL << 31) - 1) / ((K / 256) * 144))
    return fail(XQ_E_SHAPE, "one expert of rows=%lld reaches 2 GiB", (long long)rows);
  if (xrows > ((1LL << 31) - 1) / ((K / 256) * 320))
    return fail(XQ_E_SHAPE, "xq of %lld rows reaches 2 GiB", (long long)xrows);
  if ((xq::route_max_tiles(n_pairs, n_experts, 64) + xq::route_max_small_tiles(n_pairs, n_experts)) *
              ((rows + 127) / 128) + 8 > kMaxInt)
    return fail(XQ_E_SHAPE, "too many tiles for one launch");
  const size_t need = xq::gemm_q4k_id_workspace_bytes(n_pairs, n_experts);
  if (xq_status s = check_workspace(workspace, workspace_bytes, need,
                                    "xq_gemm_q4k_id_workspace_bytes"))
    return s;
  if (!aligned(y, 4)) return fail(XQ_E_ALIGN, "y not 4-byte aligned");
  if (!aligned(slab, 16)) return fail(XQ_E_ALIGN, "slab not 16-byte aligned");
  if (!aligned(xq, 16)) return fail(XQ_E_ALIGN, "xq not 16-byte aligned");
  if (!aligned(ids, 4)) return fail(XQ_E_ALIGN, "ids not 4-byte aligned");
  if (xq_status s = check_workspace_align(workspace, need)) return s;
  if (xq_status s = check_device()) return s;
  return launched(xq::launch_gemm_q4k_id(y, slab, xq, ids, n_tokens, n_used, n_experts, rows, K,
                                         static_cast<int>(x_per_slot), workspace,
                                         workspace_bytes, static_cast<hipStream_t>(stream)),
                  "xq_gemm_q4k_id");
}

size_t xq_gemm_q4k_id_workspace_bytes(int64_t n_tokens, int64_t n_used, int64_t n_experts) {
  if (n_used < 1 || n_used > kIdMaxPairs || n_tokens < 1 || n_tokens > kIdMaxPairs / n_used)
    return 0;
  return xq::gemm_q4k_id_workspace_bytes(n_tokens * n_used, n_experts);
}

xq_status xq_repack_iq4nl(void* resident, const void* file_blocks, int64_t n_blocks,
                          int64_t block_base, int64_t bpr, void* stream) {
  if (!resident) return fail(XQ_E_NULL, "resident is NULL");
  if (!file_blocks) return fail(XQ_E_NULL, "file_blocks is NULL");
  if (n_blocks < 1 || n_blocks > (1LL << 29))
    return fail(XQ_E_SHAPE, "n_blocks=%lld outside 1..2^29", (long long)n_blocks);
  if (block_base < 0 || block_base > (1LL << 40))
    return fail(XQ_E_SHAPE, "block_base=%lld outside 0..2^40", (long long)block_base);
  if (bpr < 1 || bpr > (1LL << 24))
    return fail(XQ_E_SHAPE, "bpr=%lld outside 1..2^24", (long long)bpr);
  if (!aligned(resident, 4)) return fail(XQ_E_ALIGN, "resident not 4-byte aligned");
  if (!aligned(file_blocks, 2)) return fail(XQ_E_ALIGN, "file_blocks not 2-byte aligned");
  if (xq_status s = check_device()) return s;
  return launched(xq::launch_repack_iq4nl(resident, file_blocks, n_blocks, block_base, bpr,
                                          static_cast<hipStream_t>(stream)),
                  "xq_repack_iq4nl");
}

int64_t xq_repack_dword_prefix_launches(void) { return xq::repack_dword_prefix_launches(); }

size_t xq_q8k_bytes(int64_t rows, int64_t K) {
  if (rows < 1 || K < 256 || K % 256) return 0;
  return static_cast<size_t>(rows) * static_cast<size_t>(K / 256) * 320u;
}

size_t xq_q4k_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 256 || K % 256) return 0;
  return static_cast<size_t>(N) * static_cast<size_t>(K / 256) * 144u;
}

size_t xq_iq4nl_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 256 || K % 256) return 0;
  const int64_t bpr = K / 32;
  const int64_t prefix = ((bpr * 2 + 3) / 4) * 4;
  return static_cast<size_t>(N) * static_cast<size_t>(prefix + 16 * bpr);
}

const char* xq_status_name(xq_status s) {
  switch (s) {
    case XQ_OK: return "XQ_OK";
    case XQ_E_NULL: return "XQ_E_NULL";
    case XQ_E_SHAPE: return "XQ_E_SHAPE";
    case XQ_E_ALIGN: return "XQ_E_ALIGN";
    case XQ_E_DEVICE: return "XQ_E_DEVICE";
    case XQ_E_LAUNCH: return "XQ_E_LAUNCH";
    default: return "XQ_E_UNKNOWN";
  }
}

const char* xq_last_error(void) { return g_err; }

xq_status xq_bench_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  if (!buf) return fail(XQ_E_NULL, "buf is NULL");
  if (!sink) return fail(XQ_E_NULL, "sink is NULL");
  if (bytes < 16 || bytes % 16) return fail(XQ_E_SHAPE, "bytes=%lld not a positive multiple of 16", (long long)bytes);
  if (!aligned(buf, 16)) return fail(XQ_E_ALIGN, "buf not 16-byte aligned");
  if (!aligned(sink, 4)) return fail(XQ_E_ALIGN, "sink not 4-byte aligned");
  if (xq_status s = check_device()) return s;
  return launched(xq::launch_stream_read(buf, bytes, sink, static_cast<hipStream_t>(stream)),
                  "xq_bench_stream_read");
}

int64_t xq_bench_sink_words(int64_t bytes) { return xq::stream_read_sink_words(bytes); }

}  // extern "C"
