// C ABI of liblowbit: argument validation, dispatch and the per-stream
// workspace.  Every check runs on the host before any HIP call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/lowbit.h"
#include "common.hpp"

using namespace lowbit;

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool valid_fmt(int fmt) {
  return fmt == LOWBIT_BINARY || fmt == LOWBIT_TERNARY_2BIT || fmt == LOWBIT_TERNARY_BASE3;
}

// N * K and derived sizes must stay far from int64 overflow
bool shape_ok(int64_t N, int64_t K) {
  if (N < 1 || K < 1 || K % kGroup != 0) return false;
  if (N > (int64_t(1) << 40) || K > (int64_t(1) << 40)) return false;
  if (N > (int64_t(1) << 62) / K) return false;
  return true;
}

int hip_status(hipError_t e) { return e == hipSuccess ? LOWBIT_OK : LOWBIT_E_HIP; }

// ---- per-(device, stream) workspace, grown on demand.  A grown workspace
// serves the stream's later calls; the smaller one it replaces is retired,
// not freed, because kernels queued before the growth, and HIP graphs
// captured on the stream, may still use it.  Nothing waits for the stream.
// A stream being captured cannot grow its workspace (reserve it first).
// Retired and current workspaces are freed by lowbit_release_workspaces.
// The first kCounterBytes of a workspace hold the kernels' arrival counters
// (zeroed on the stream when the workspace is allocated; every launch leaves
// them zero).
struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
std::vector<std::pair<int, void*>> g_retired;  // (device, workspace)

int workspace(hipStream_t s, size_t need, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LOWBIT_E_HIP;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  Workspace& w = g_ws[{dev, s}];
  if (w.bytes < need) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) return LOWBIT_E_HIP;
    if (cs != hipStreamCaptureStatusNone) return LOWBIT_E_NOMEM;
    const size_t sz = need < (1u << 20) ? (1u << 20) : need + need / 4;
    void* p = nullptr;
    if (hipMalloc(&p, sz) != hipSuccess) return LOWBIT_E_NOMEM;
    // the counter block must start at zero; kernels leave it zero
    if (hipMemsetAsync(p, 0, kCounterBytes, s) != hipSuccess) {
      (void)hipFree(p);
      return LOWBIT_E_HIP;
    }
    if (w.ptr) g_retired.push_back({dev, w.ptr});
    w.ptr = p;
    w.bytes = sz;
  }
  *out = w.ptr;
  return LOWBIT_OK;
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---- the allocation-free GEMV's scratch: one static device array per GPU,
// shared by every lowbit_gemv_noalloc call on that GPU.  Host code uses only
// the device address hipGetSymbolAddress returns for the current device
// (taken once per device, under g_scratch_mutex); the array's name on the
// host is not a device address.  Its first kCounterBytes hold the fused
// GEMV's arrival counters: zero when the code object is loaded (static
// storage), cleared again by a fill kernel on the first call's stream, and
// left zero by every launch.
constexpr size_t kScratchBytes = size_t(4) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
static_assert(kScratchBytes >= (size_t)kCounterBytes, "counters must fit the scratch");

__global__ void fill_zero_u32(uint32_t* p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

std::mutex g_scratch_mutex;
std::map<int, void*> g_scratch;  // device -> address of `scratch` on it

int scratch_for_device(hipStream_t s, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LOWBIT_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  auto it = g_scratch.find(dev);
  if (it == g_scratch.end()) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return LOWBIT_E_HIP;
    hipLaunchKernelGGL(fill_zero_u32, dim3(64), dim3(256), 0, s, (uint32_t*)ptr,
                       (int64_t)(kCounterBytes / 4));
    if (hipGetLastError() != hipSuccess) return LOWBIT_E_HIP;
    it = g_scratch.emplace(dev, ptr).first;
  }
  *out = it->second;
  return LOWBIT_OK;
}

// small-M product through the fused MFMA GEMV kernel (M * R <= 16 rows of A)
// with the workspace `ws` (counters first, zero)
int gemv_mfma_ws(int fmt, int64_t M, int64_t N, int64_t K, const void* pcodes,
                 const void* pscales, int x_dtype, const void* x, float x_scale,
                 const float* x_scales, int y_dtype, void* y, void* ws, hipStream_t s) {
  GemvArgs g;
  g.fmt = fmt;
  g.N = N;
  g.K = K;
  g.M = M;
  g.pcodes = pcodes;
  g.pscales = (const uint16_t*)pscales;
  g.xkind = x_dtype;
  g.x = x;
  g.x_scale = (x_dtype == LOWBIT_I8) ? x_scale : 1.0f;
  g.x_scales = x_scales;
  g.ykind = y_dtype;
  g.y = y;
  g.ws = ws;
  return hip_status(launch_gemv_mfma(g, s));
}

int run_gemv_mfma(int fmt, int64_t M, int64_t N, int64_t K, const void* pcodes,
                  const void* pscales, int x_dtype, const void* x, float x_scale,
                  const float* x_scales, int y_dtype, void* y, hipStream_t s) {
  if (cdiv(N, 16) > kMaxRowGroups) return LOWBIT_E_SHAPE;
  void* ws = nullptr;
  int rc = workspace(s, gemv_workspace_bytes(fmt, N, K, M, x_dtype), &ws);
  if (rc) return rc;
  return gemv_mfma_ws(fmt, M, N, K, pcodes, pscales, x_dtype, x, x_scale, x_scales, y_dtype, y,
                      ws, s);
}

// large-M product through the staged-tile MFMA GEMM
int run_gemm(int fmt, int64_t M, int64_t N, int64_t K, const void* pcodes, const void* pscales,
             int x_dtype, const void* X, const float* x_scales, int y_dtype, void* Y,
             hipStream_t s) {
  if (cdiv(N, 16) > (int64_t(1) << 40) / 16) return LOWBIT_E_SHAPE;
  void* ws = nullptr;
  int rc = workspace(s, gemm_workspace_bytes(fmt, x_dtype, M, N, K), &ws);
  if (rc) return rc;
  GemmArgs g;
  g.fmt = fmt;
  g.M = M;
  g.N = N;
  g.K = K;
  g.pcodes = pcodes;
  g.pscales = (const uint16_t*)pscales;
  g.xkind = x_dtype;
  g.x = X;
  g.x_scales = x_dtype != LOWBIT_BF16 && y_dtype != LOWBIT_I32 ? x_scales : nullptr;
  g.ykind = y_dtype;
  g.y = Y;
  g.ws = ws;
  return hip_status(launch_gemm(g, s));
}

// activation rows the batch-1 kernels take at once: 16 rows of A over the
// split terms of one row
int max_small_m(int fmt, int x_dtype) { return 16 / split_terms(fmt, x_dtype); }

// Workspace bytes a product needs: the path lowbit_gemm (or lowbit_gemv when
// M = 1) takes for these arguments.  Sign activations: the GEMM's need (the
// batch-1 sign GEMV of lowbit_gemv uses none, so this bounds both).
size_t product_workspace(int fmt, int64_t M, int64_t N, int64_t K, int x_dtype) {
  if (x_dtype != LOWBIT_SIGN1 && M <= max_small_m(fmt, x_dtype))
    return gemv_workspace_bytes(fmt, N, K, M, x_dtype);
  return gemm_workspace_bytes(fmt, x_dtype, M, N, K);
}

}  // namespace

extern "C" {

int lowbit_abi_version(void) { return LOWBIT_ABI_VERSION; }

const char* lowbit_status_str(int status) {
  switch (status) {
    case LOWBIT_OK: return "ok";
    case LOWBIT_E_NULL: return "null pointer";
    case LOWBIT_E_SHAPE: return "invalid shape (K must be a positive multiple of 128)";
    case LOWBIT_E_ALIGN: return "misaligned pointer";
    case LOWBIT_E_UNSUPPORTED: return "unsupported format / dtype combination";
    case LOWBIT_E_BADCODE: return "invalid code";
    case LOWBIT_E_HIP: return "HIP runtime error";
    case LOWBIT_E_NOMEM: return "workspace allocation failed (or needed growth during graph capture)";
    case LOWBIT_E_TOO_LARGE: return "product needs more scratch than the allocation-free call holds";
  }
  return "unknown status";
}

int lowbit_packed_bytes(int fmt, int64_t N, int64_t K, size_t* code_bytes, size_t* scale_bytes) {
  if (!code_bytes || !scale_bytes) return LOWBIT_E_NULL;
  if (!valid_fmt(fmt)) return LOWBIT_E_UNSUPPORTED;
  if (!shape_ok(N, K)) return LOWBIT_E_SHAPE;
  int64_t NB = cdiv(N, 16), G = K / kGroup;
  int64_t c = fmt == LOWBIT_BINARY ? NB * cdiv(G, 4) * 1024
              : fmt == LOWBIT_TERNARY_2BIT ? NB * cdiv(G, 2) * 1024
                                           : NB * cdiv(G, 8) * 3328;
  *code_bytes = (size_t)c;
  *scale_bytes = (size_t)(NB * cdiv(G, 4) * 128);
  return LOWBIT_OK;
}

int lowbit_pack(int fmt, int64_t N, int64_t K, const int8_t* codes, const uint16_t* scales,
                void* pcodes, void* pscales, int32_t* bad_code_count, void* stream) {
  if (!codes || !scales || !pcodes || !pscales) return LOWBIT_E_NULL;
  if (!valid_fmt(fmt)) return LOWBIT_E_UNSUPPORTED;
  if (!shape_ok(N, K)) return LOWBIT_E_SHAPE;
  if (!aligned(pcodes, 16) || !aligned(pscales, 16) || !aligned(scales, 2) ||
      (bad_code_count && !aligned(bad_code_count, 4)))
    return LOWBIT_E_ALIGN;
  return hip_status(launch_pack(fmt, N, K, codes, scales, pcodes, pscales, bad_code_count,
                                (hipStream_t)stream));
}

int lowbit_unpack(int fmt, int64_t N, int64_t K, const void* pcodes, const void* pscales,
                  int8_t* codes, uint16_t* scales, int32_t* bad_code_count, void* stream) {
  if (!codes || !scales || !pcodes || !pscales) return LOWBIT_E_NULL;
  if (!valid_fmt(fmt)) return LOWBIT_E_UNSUPPORTED;
  if (!shape_ok(N, K)) return LOWBIT_E_SHAPE;
  if (!aligned(pcodes, 16) || !aligned(pscales, 16) || !aligned(scales, 2) ||
      (bad_code_count && !aligned(bad_code_count, 4)))
    return LOWBIT_E_ALIGN;
  return hip_status(launch_unpack(fmt, N, K, pcodes, pscales, codes, scales, bad_code_count,
                                  (hipStream_t)stream));
}

int lowbit_quantize_act_i8(int64_t M, int64_t K, const uint16_t* X_bf16, int8_t* Q, float* s_x,
                           void* stream) {
  if (!X_bf16 || !Q || !s_x) return LOWBIT_E_NULL;
  if (M < 1 || K < 1 || M > (int64_t(1) << 31) || K > (int64_t(1) << 40)) return LOWBIT_E_SHAPE;
  if (!aligned(X_bf16, 2) || !aligned(s_x, 4)) return LOWBIT_E_ALIGN;
  return hip_status(launch_quantize_i8(M, K, X_bf16, Q, s_x, (hipStream_t)stream));
}

namespace {

// argument checks of lowbit_gemv (and its allocation-free variant)
int gemv_check(int fmt, int64_t N, int64_t K, const void* pcodes, const void* pscales,
               int x_dtype, const void* x, int y_dtype, void* y) {
  if (!pcodes || !x || !y) return LOWBIT_E_NULL;
  if (!valid_fmt(fmt)) return LOWBIT_E_UNSUPPORTED;
  if (!shape_ok(N, K)) return LOWBIT_E_SHAPE;
  const bool int_x = x_dtype == LOWBIT_I8 || x_dtype == LOWBIT_SIGN1;
  if (x_dtype < LOWBIT_F32 || x_dtype > LOWBIT_SIGN1) return LOWBIT_E_UNSUPPORTED;
  if (y_dtype != LOWBIT_F32 && y_dtype != LOWBIT_BF16 && y_dtype != LOWBIT_I32)
    return LOWBIT_E_UNSUPPORTED;
  if (y_dtype == LOWBIT_I32 && !(int_x && pscales == nullptr)) return LOWBIT_E_UNSUPPORTED;
  if (y_dtype != LOWBIT_I32 && !pscales) return LOWBIT_E_NULL;
  if (x_dtype == LOWBIT_SIGN1 && fmt != LOWBIT_BINARY) return LOWBIT_E_UNSUPPORTED;
  if (!aligned(pcodes, 16) || (pscales && !aligned(pscales, 16)) || !aligned(x, 16) ||
      !aligned(y, 4))
    return LOWBIT_E_ALIGN;
  if (x_dtype == LOWBIT_SIGN1 && K > kSignMaxK) return LOWBIT_E_SHAPE;  // sign words in LDS
  if (x_dtype != LOWBIT_SIGN1 && cdiv(N, 16) > kMaxRowGroups) return LOWBIT_E_SHAPE;
  return LOWBIT_OK;
}

int gemv_sign(int64_t N, int64_t K, const void* pcodes, const void* pscales, const void* x,
              float x_scale, int y_dtype, void* y, hipStream_t s) {
  SignArgs a;
  a.N = N;
  a.K = K;
  a.M = 1;
  a.pcodes = pcodes;
  a.pscales = (const uint16_t*)pscales;
  a.xbits = (const uint8_t*)x;
  a.alpha = x_scale;
  a.ykind = y_dtype;
  a.y = y;
  return hip_status(launch_gemv_sign(a, s));
}

}  // namespace

int lowbit_gemv(int fmt, int64_t N, int64_t K, const void* pcodes, const void* pscales,
                int x_dtype, const void* x, float x_scale, int y_dtype, void* y, void* stream) {
  const int rc = gemv_check(fmt, N, K, pcodes, pscales, x_dtype, x, y_dtype, y);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  if (x_dtype == LOWBIT_SIGN1) return gemv_sign(N, K, pcodes, pscales, x, x_scale, y_dtype, y, s);
  return run_gemv_mfma(fmt, 1, N, K, pcodes, pscales, x_dtype, x, x_scale, nullptr, y_dtype, y,
                       s);
}

int lowbit_gemv_noalloc(int fmt, int64_t N, int64_t K, const void* pcodes, const void* pscales,
                        int x_dtype, const void* x, float x_scale, int y_dtype, void* y,
                        void* stream) {
  const int rc = gemv_check(fmt, N, K, pcodes, pscales, x_dtype, x, y_dtype, y);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  if (x_dtype == LOWBIT_SIGN1) return gemv_sign(N, K, pcodes, pscales, x, x_scale, y_dtype, y, s);
  if (gemv_workspace_bytes(fmt, N, K, 1, x_dtype) > kScratchBytes) return LOWBIT_E_TOO_LARGE;
  void* ws = nullptr;
  const int r2 = scratch_for_device(s, &ws);
  if (r2) return r2;
  return gemv_mfma_ws(fmt, 1, N, K, pcodes, pscales, x_dtype, x, x_scale, nullptr, y_dtype, y, ws,
                      s);
}

int lowbit_gemm(int fmt, int64_t M, int64_t N, int64_t K, const void* pcodes, const void* pscales,
                int x_dtype, const void* X, const float* x_scales, int y_dtype, void* Y,
                void* stream) {
  if (!pcodes || !X || !Y) return LOWBIT_E_NULL;
  if (!valid_fmt(fmt)) return LOWBIT_E_UNSUPPORTED;
  if (!shape_ok(N, K) || M < 1 || M > (int64_t(1) << 31)) return LOWBIT_E_SHAPE;
  if (K > (int64_t(1) << 36)) return LOWBIT_E_SHAPE;  // 32-bit group indices of the GEMM
  const bool sign = x_dtype == LOWBIT_SIGN1;
  if (x_dtype != LOWBIT_BF16 && x_dtype != LOWBIT_I8 && !sign) return LOWBIT_E_UNSUPPORTED;
  if (y_dtype != LOWBIT_F32 && y_dtype != LOWBIT_BF16 && y_dtype != LOWBIT_I32)
    return LOWBIT_E_UNSUPPORTED;
  if (y_dtype == LOWBIT_I32 && !((x_dtype == LOWBIT_I8 || sign) && pscales == nullptr))
    return LOWBIT_E_UNSUPPORTED;
  if (y_dtype != LOWBIT_I32 && !pscales) return LOWBIT_E_NULL;
  if ((x_dtype == LOWBIT_I8 || sign) && y_dtype != LOWBIT_I32 && !x_scales) return LOWBIT_E_NULL;
  if (!aligned(pcodes, 16) || (pscales && !aligned(pscales, 16)) || !aligned(X, 16) ||
      !aligned(Y, 16) || (x_scales && !aligned(x_scales, 4)))
    return LOWBIT_E_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  if (!sign && M <= max_small_m(fmt, x_dtype))
    return run_gemv_mfma(fmt, M, N, K, pcodes, pscales, x_dtype, X, 1.0f,
                         x_dtype == LOWBIT_I8 && y_dtype != LOWBIT_I32 ? x_scales : nullptr,
                         y_dtype, Y, s);
  return run_gemm(fmt, M, N, K, pcodes, pscales, x_dtype, X, x_scales, y_dtype, Y, s);
}

int lowbit_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K, int x_dtype, size_t* bytes) {
  if (!bytes) return LOWBIT_E_NULL;
  *bytes = 0;
  if (!valid_fmt(fmt)) return LOWBIT_E_UNSUPPORTED;
  if (x_dtype < LOWBIT_F32 || x_dtype > LOWBIT_SIGN1) return LOWBIT_E_UNSUPPORTED;
  if (!shape_ok(N, K) || M < 1 || M > (int64_t(1) << 31) || K > (int64_t(1) << 36))
    return LOWBIT_E_SHAPE;
  if (M > 1 && x_dtype == LOWBIT_F32) return LOWBIT_E_UNSUPPORTED;  // lowbit_gemm takes no F32
  *bytes = product_workspace(fmt, M, N, K, x_dtype);
  return LOWBIT_OK;
}

int lowbit_reserve_workspace(size_t bytes, void* stream) {
  void* ws = nullptr;
  return workspace((hipStream_t)stream, bytes, &ws);
}

int lowbit_release_workspaces(void) {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  int rc = LOWBIT_OK;
  int cur = 0;
  if (!g_ws.empty() || !g_retired.empty())
    if (hipGetDevice(&cur) != hipSuccess) return LOWBIT_E_HIP;
  std::vector<int> devs;
  for (auto& kv : g_ws) devs.push_back(kv.first.first);
  for (auto& r : g_retired) devs.push_back(r.first);
  std::sort(devs.begin(), devs.end());
  devs.erase(std::unique(devs.begin(), devs.end()), devs.end());
  for (int d : devs)  // queued kernels may still use a workspace
    if (hipSetDevice(d) != hipSuccess || hipDeviceSynchronize() != hipSuccess) rc = LOWBIT_E_HIP;
  auto release = [&](int dev, void* p) {
    if (hipSetDevice(dev) != hipSuccess || hipFree(p) != hipSuccess) rc = LOWBIT_E_HIP;
  };
  for (auto& kv : g_ws)
    if (kv.second.ptr) release(kv.first.first, kv.second.ptr);
  for (auto& r : g_retired) release(r.first, r.second);
  g_ws.clear();
  g_retired.clear();
  if (rc == LOWBIT_OK && hipSetDevice(cur) != hipSuccess) rc = LOWBIT_E_HIP;
  return rc;
}

struct lowbit_chain {
  void* plan;
};

int lowbit_chain_create_rows(int n_stages, const lowbit_gemv_stage* stages, int64_t rows,
                             int x_dtype, int y_dtype, lowbit_chain** chain) {
  if (!stages || !chain) return LOWBIT_E_NULL;
  *chain = nullptr;
  if (n_stages < 1) return LOWBIT_E_SHAPE;
  if (x_dtype != LOWBIT_F32 && x_dtype != LOWBIT_BF16) return LOWBIT_E_UNSUPPORTED;
  if (y_dtype != LOWBIT_F32 && y_dtype != LOWBIT_BF16) return LOWBIT_E_UNSUPPORTED;
  const int fmt = stages[0].fmt;
  if (!valid_fmt(fmt)) return LOWBIT_E_UNSUPPORTED;
  if (rows < 1 || rows > max_small_m(fmt, x_dtype)) return LOWBIT_E_SHAPE;
  std::vector<ChainStage> st(n_stages);
  for (int i = 0; i < n_stages; i++) {
    const lowbit_gemv_stage& g = stages[i];
    if (g.fmt != fmt) return LOWBIT_E_UNSUPPORTED;
    if (!g.pcodes || !g.pscales || !g.x || !g.y) return LOWBIT_E_NULL;
    if (!shape_ok(g.N, g.K) || cdiv(g.N, 16) > kMaxRowGroups) return LOWBIT_E_SHAPE;
    // a waiting stage reads x through a buffer descriptor (32-bit byte offsets)
    if (i > 0 && g.wait_prev && rows * g.K * (x_dtype == LOWBIT_F32 ? 4 : 2) > INT32_MAX)
      return LOWBIT_E_SHAPE;
    if (!aligned(g.pcodes, 16) || !aligned(g.pscales, 16) || !aligned(g.x, 16) || !aligned(g.y, 4))
      return LOWBIT_E_ALIGN;
    if (g.epilogue != LOWBIT_EPI_NONE && g.epilogue != LOWBIT_EPI_SILU_MUL) return LOWBIT_E_UNSUPPORTED;
    if (g.epilogue == LOWBIT_EPI_SILU_MUL && (g.N % 16 != 0 || rows != 1)) return LOWBIT_E_SHAPE;
    st[i] = ChainStage{fmt, g.N, g.K, g.pcodes, (const uint16_t*)g.pscales, g.x, g.y,
                       i > 0 && g.wait_prev ? 1 : 0, g.epilogue};
  }
  void* plan = nullptr;
  hipError_t e = chain_create(st.data(), n_stages, rows, x_dtype, y_dtype, &plan);
  if (e == hipErrorOutOfMemory) return LOWBIT_E_NOMEM;
  if (e != hipSuccess) return LOWBIT_E_HIP;
  *chain = new lowbit_chain{plan};
  return LOWBIT_OK;
}

int lowbit_chain_create(int n_stages, const lowbit_gemv_stage* stages, int x_dtype, int y_dtype,
                        lowbit_chain** chain) {
  return lowbit_chain_create_rows(n_stages, stages, 1, x_dtype, y_dtype, chain);
}

int lowbit_chain_run(lowbit_chain* chain, void* stream) {
  if (!chain) return LOWBIT_E_NULL;
  return hip_status(chain_run(chain->plan, (hipStream_t)stream));
}

int lowbit_chain_status(lowbit_chain* chain, int* failed_waits) {
  if (!chain || !failed_waits) return LOWBIT_E_NULL;
  return hip_status(chain_status(chain->plan, failed_waits));
}

int lowbit_chain_destroy(lowbit_chain* chain) {
  if (!chain) return LOWBIT_OK;
  const hipError_t e = hipDeviceSynchronize();
  chain_destroy(chain->plan);
  delete chain;
  return hip_status(e);
}

}  // extern "C"

int lowbit_hbm_read_probe(const void* src, int64_t bytes, uint32_t* out, void* stream) {
  if (!src || !out) return LOWBIT_E_NULL;
  if (bytes < 16 || bytes % 16 != 0) return LOWBIT_E_SHAPE;
  if (!aligned(src, 16) || !aligned(out, 4)) return LOWBIT_E_ALIGN;
  return hip_status(launch_hbm_read(src, bytes, out, (hipStream_t)stream));
}

int lowbit_quantize_weights(int fmt, int64_t N, int64_t K, const uint16_t* W_bf16,
                            const int8_t* signs, int8_t* codes, uint16_t* scales, void* stream) {
  if (!W_bf16 || !codes || !scales) return LOWBIT_E_NULL;
  if (!valid_fmt(fmt)) return LOWBIT_E_UNSUPPORTED;
  if (!shape_ok(N, K)) return LOWBIT_E_SHAPE;
  if (!aligned(W_bf16, 16) || !aligned(codes, 16) || (signs && !aligned(signs, 16)) ||
      !aligned(scales, 2))
    return LOWBIT_E_ALIGN;
  return hip_status(launch_quantize_weights(fmt, N, K, W_bf16, signs, codes, scales,
                                            (hipStream_t)stream));
}

int lowbit_rotate_act(int64_t M, int64_t K, const uint16_t* X_bf16, const int8_t* signs,
                      float* X_rot, void* stream) {
  if (!X_bf16 || !signs || !X_rot) return LOWBIT_E_NULL;
  if (!shape_ok(M, K)) return LOWBIT_E_SHAPE;
  if (!aligned(X_bf16, 2) || !aligned(X_rot, 4)) return LOWBIT_E_ALIGN;
  return hip_status(launch_rotate_act(M, K, X_bf16, signs, X_rot, (hipStream_t)stream));
}

