// api.hip -- the extern "C" boundary of libmhc (declared in include/mhc.h).
//
// Every entry point validates all of its arguments on the host before it
// enqueues anything (fail closed), then launches on the caller's stream.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/mhc.h"
#include "internal.h"

namespace {

thread_local std::string g_last_error;

// mhc_set_kernel_events registration, per host thread
struct KernelEvents {
  int kernel = 0;
  hipEvent_t start = nullptr, stop = nullptr;
};
thread_local KernelEvents g_kernel_events;

struct Span {
  const char *name;
  uintptr_t lo, hi;
};

// Collects the buffers of one call and checks them.
class Validator {
 public:
  explicit Validator(const char *fn) : fn_(fn) {}

  bool ok() const { return st_ == MHC_OK; }
  mhc_status status() const { return st_; }

  void fail(mhc_status s, const std::string &msg) {
    if (st_ != MHC_OK) return;
    st_ = s;
    g_last_error = std::string(fn_) + ": " + msg;
  }

  void dims(int64_t tokens, int32_t n, int64_t C, mhc_dtype act) {
    if (tokens < 0) fail(MHC_ERR_SHAPE, "tokens must be >= 0");
    if (tokens > mhc::kMaxTokens) fail(MHC_ERR_UNSUPPORTED, "tokens must be <= 4194304");
    if (n <= 0) fail(MHC_ERR_SHAPE, "n must be > 0");
    if (C <= 0) fail(MHC_ERR_SHAPE, "C must be > 0");
    if (n > mhc::kMaxN) fail(MHC_ERR_UNSUPPORTED, "n must be <= 8");
    if (C > 0 && C % 8 != 0) fail(MHC_ERR_UNSUPPORTED, "C must be a multiple of 8");
    if (C > mhc::kMaxC) fail(MHC_ERR_UNSUPPORTED, "C must be <= 16384");
    if (act != MHC_BF16 && act != MHC_F32) fail(MHC_ERR_ARG, "unknown activation dtype");
  }

  // [tokens][C] rows with no stream dimension (the RMSNorm of the aggregated stream)
  void rows(int64_t tokens, int64_t C, mhc_dtype act) { dims(tokens, 1, C, act); }

  void eps(float e, const char *what) {
    if (!std::isfinite(e) || e < 0.f) fail(MHC_ERR_ARG, std::string(what) + " must be finite and >= 0");
  }

  // matrix count of the Sinkhorn entry points
  void count(int64_t c) {
    if (c < 0) fail(MHC_ERR_SHAPE, "count must be >= 0");
    if (c > mhc::kMaxTokens) fail(MHC_ERR_UNSUPPORTED, "count must be <= 4194304");
  }

  void iters(int32_t it) {
    if (it < 0) fail(MHC_ERR_ARG, "iters must be >= 0");
    if (it > 4096) fail(MHC_ERR_UNSUPPORTED, "iters must be <= 4096");
  }

  // A device buffer of `bytes` bytes.  Optional buffers may be NULL.
  void in(const void *p, size_t bytes, const char *name, bool optional = false) {
    add(p, bytes, name, optional, ins_);
  }
  void out(const void *p, size_t bytes, const char *name, bool optional = false) {
    add(p, bytes, name, optional, outs_);
  }

  void workspace(const void *ws, size_t have, size_t need) {
    if (need == 0) return;
    if (!ws) { fail(MHC_ERR_WORKSPACE, "workspace is NULL but " + std::to_string(need) + " bytes are needed"); return; }
    if (have < need) {
      fail(MHC_ERR_WORKSPACE, "workspace too small: " + std::to_string(have) + " < " + std::to_string(need));
      return;
    }
    if (reinterpret_cast<uintptr_t>(ws) % 16) { fail(MHC_ERR_ALIGN, "workspace not 16-byte aligned"); return; }
    outs_.push_back({"workspace", reinterpret_cast<uintptr_t>(ws), reinterpret_cast<uintptr_t>(ws) + need});
  }

  // Outputs must not overlap inputs or each other.
  mhc_status finish() {
    if (st_ != MHC_OK) return st_;
    for (size_t a = 0; a < outs_.size(); ++a) {
      for (const Span &b : ins_)
        if (overlap(outs_[a], b)) {
          fail(MHC_ERR_ALIAS, std::string(outs_[a].name) + " overlaps input " + b.name);
          return st_;
        }
      for (size_t b = a + 1; b < outs_.size(); ++b)
        if (overlap(outs_[a], outs_[b])) {
          fail(MHC_ERR_ALIAS, std::string(outs_[a].name) + " overlaps output " + outs_[b].name);
          return st_;
        }
    }
    return st_;
  }

 private:
  static bool overlap(const Span &a, const Span &b) { return a.lo < b.hi && b.lo < a.hi; }

  void add(const void *p, size_t bytes, const char *name, bool optional, std::vector<Span> &v) {
    if (!p) {
      if (!optional) fail(MHC_ERR_NULL, std::string(name) + " is NULL");
      return;
    }
    if (reinterpret_cast<uintptr_t>(p) % 16) {
      fail(MHC_ERR_ALIGN, std::string(name) + " is not 16-byte aligned");
      return;
    }
    if (bytes) v.push_back({name, reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + bytes});
  }

  const char *fn_;
  mhc_status st_ = MHC_OK;
  std::vector<Span> ins_, outs_;
};

inline size_t esz(mhc_dtype act) { return act == MHC_F32 ? 4 : 2; }

mhc_status launched(const char *fn) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    g_last_error = std::string(fn) + ": launch failed: " + hipGetErrorString(e);
    return MHC_ERR_HIP;
  }
  return MHC_OK;
}

__global__ void fill_zero_kernel(float *p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

__global__ void fill_zero_u16_kernel(uint16_t *p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Zero-fill kernels (not hipMemsetAsync, so callers may capture the call in
// a HIP graph).  Return whether anything was launched.
bool zero_f32(hipStream_t s, float *p, int64_t n) {
  if (!p || n <= 0) return false;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
  return true;
}

__global__ void copy16_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst, int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n16) dst[i] = src[i];
}

// dst = src, `bytes` a multiple of 16 (a kernel, not a copy node, so callers may capture the call)
void copy16(hipStream_t s, const void *src, void *dst, int64_t bytes) {
  const int64_t n16 = bytes / 16;
  if (n16 <= 0) return;
  hipLaunchKernelGGL(copy16_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s, (const uint4 *)src,
                     (uint4 *)dst, n16);
}

bool zero_act(hipStream_t s, void *p, int64_t n, mhc_dtype act) {
  if (!p || n <= 0) return false;
  if (act == MHC_F32) return zero_f32(s, (float *)p, n);
  hipLaunchKernelGGL(fill_zero_u16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (uint16_t *)p, n);
  return true;
}


// ---- fused pre forward: checks and launches shared by mhc_pre_fwd and mhc_pre_fwd_noalloc
size_t pre_fwd_ws(int64_t tokens, int32_t n, int64_t C, mhc_dtype act) {
  return n == 4 ? mhc::proj_fwd_ws(tokens, C, act == MHC_F32)
                : mhc::gproj_fwd_ws(n, tokens, C, act == MHC_F32);
}

// Shapes, scalars and every tensor argument (no workspace).  False when a check failed or
// tokens == 0 (then v.status() is the result).
bool pre_fwd_check(Validator &v, int64_t tokens, int32_t n, int64_t C, mhc_dtype act, const void *X,
                   const float *W, const float *alpha, const float *hbias, float rms_eps, int32_t iters,
                   float eps, float *H_pre, float *H_post, float *H_res, float *H_res_logits, float *saved,
                   void *agg) {
  v.dims(tokens, n, C, act);
  v.eps(rms_eps, "rms_eps");
  v.eps(eps, "eps");
  v.iters(iters);
  if (!v.ok()) return false;
  if (tokens == 0) return true;
  const int64_t K = (int64_t)n * C;
  const int64_t J = (int64_t)n * n + 2 * n;
  v.in(X, tokens * K * esz(act), "X");
  v.in(W, K * J * 4, "W");
  v.in(alpha, 12, "alpha", true);
  v.in(hbias, J * 4, "hbias", true);
  v.out(H_pre, tokens * n * 4, "H_pre");
  v.out(H_post, tokens * n * 4, "H_post");
  v.out(H_res, tokens * n * n * 4, "H_res");
  v.out(H_res_logits, tokens * n * n * 4, "H_res_logits");
  v.out(saved, tokens * mhc::saved_stride(n) * 4, "saved", true);
  v.out(agg, tokens * C * esz(act), "agg");
  return v.ok();
}

void pre_fwd_launch(hipStream_t s, int64_t tokens, int32_t n, int64_t C, mhc_dtype act, const void *X,
                    const float *W, const float *alpha, const float *hbias, float rms_eps, int32_t iters,
                    float eps, float *H_pre, float *H_post, float *H_res, float *H_res_logits, float *saved,
                    void *agg, void *ws) {
  if (n == 4) {
    mhc::launch_proj_fwd(s, act == MHC_F32, tokens, C, X, W, alpha, hbias, rms_eps, H_pre, H_post,
                         H_res_logits, saved, H_res, iters, eps, ws);
    mhc::launch_h_aggregate_fwd(s, act == MHC_F32, tokens, C, X, H_pre, agg);
  } else {
    mhc::glaunch_proj_fwd(s, act == MHC_F32, n, tokens, C, X, W, alpha, hbias, rms_eps, H_pre, H_post,
                          H_res_logits, saved, H_res, iters, eps, ws);
    mhc::glaunch_h_aggregate_fwd(s, act == MHC_F32, n, tokens, C, X, H_pre, agg, n);
  }
}

}  // namespace

// ---- the static scratch of mhc_pre_fwd_noalloc
// One array of MHC_NOALLOC_SCRATCH_BYTES in device memory: every GPU that
// loads this library holds its own copy, at its own address, until the
// process ends.  In host code `scratch` names a host-side stand-in, never
// the device memory: the device address comes from hipGetSymbolAddress,
// looked up once per device with that device current, and only that
// address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[MHC_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices];  // device address of `scratch` per device id, once looked up

// Device address of the current device's scratch array (looked up on the first call per device).
mhc_status scratch_of_current_device(void **addr, const char *fn) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_error = std::string(fn) + ": hipGetDevice failed: " + hipGetErrorString(e);
    return MHC_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    g_last_error = std::string(fn) + ": device id " + std::to_string(dev) + " out of range";
    return MHC_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      g_last_error = std::string(fn) + ": hipGetSymbolAddress(scratch) failed: " + hipGetErrorString(e);
      return MHC_ERR_HIP;
    }
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return MHC_OK;
}

}  // namespace

static_assert(mhc::kKernelProjBwdDxDw == MHC_KERNEL_PROJ_BWD_DXDW, "kernel ids");

void mhc::kernel_event(int id, hipStream_t s, bool start) {
  const KernelEvents &k = g_kernel_events;
  if (k.kernel != id) return;
  (void)hipEventRecord(start ? k.start : k.stop, s);
}

extern "C" {

const char *mhc_status_string(mhc_status s) {
  switch (s) {
    case MHC_OK: return "MHC_OK";
    case MHC_ERR_NULL: return "MHC_ERR_NULL";
    case MHC_ERR_SHAPE: return "MHC_ERR_SHAPE";
    case MHC_ERR_UNSUPPORTED: return "MHC_ERR_UNSUPPORTED";
    case MHC_ERR_ALIGN: return "MHC_ERR_ALIGN";
    case MHC_ERR_ALIAS: return "MHC_ERR_ALIAS";
    case MHC_ERR_WORKSPACE: return "MHC_ERR_WORKSPACE";
    case MHC_ERR_ARG: return "MHC_ERR_ARG";
    case MHC_ERR_HIP: return "MHC_ERR_HIP";
  }
  return "MHC_ERR_UNKNOWN";
}

const char *mhc_last_error(void) { return g_last_error.c_str(); }

const char *mhc_version(void) { return "libmhc 0.1 gfx950"; }

int32_t mhc_saved_stride(int32_t n) { return (n < 1 || n > mhc::kMaxN) ? 0 : mhc::saved_stride(n); }

mhc_status mhc_set_kernel_events(int32_t kernel, void *start_event, void *stop_event) {
  if (kernel == MHC_KERNEL_NONE || (!start_event && !stop_event)) {
    g_kernel_events = KernelEvents{};
    return MHC_OK;
  }
  if (kernel != MHC_KERNEL_PROJ_BWD_DXDW) {
    g_last_error = "mhc_set_kernel_events: unknown kernel id " + std::to_string(kernel);
    return MHC_ERR_ARG;
  }
  if (!start_event || !stop_event) {
    g_last_error = "mhc_set_kernel_events: start_event and stop_event must both be set or both be NULL";
    return MHC_ERR_ARG;
  }
  g_kernel_events = KernelEvents{kernel, (hipEvent_t)start_event, (hipEvent_t)stop_event};
  return MHC_OK;
}

mhc_status mhc_bandwidth_probe(void *stream, int32_t kind, const void *src, void *dst, size_t bytes) {
  Validator v("mhc_bandwidth_probe");
  const bool copy = (kind & MHC_PROBE_COPY) != 0;
  if (kind < 0 || kind > (MHC_PROBE_COPY | MHC_PROBE_NONTEMPORAL)) v.fail(MHC_ERR_ARG, "unknown probe kind");
  if (bytes % 16) v.fail(MHC_ERR_SHAPE, "bytes must be a multiple of 16");
  if (bytes > ((size_t)1 << 40)) v.fail(MHC_ERR_UNSUPPORTED, "bytes must be <= 2^40");
  if (!v.ok()) return v.status();
  if (bytes == 0) return MHC_OK;
  v.in(src, bytes, "src");
  v.out(dst, copy ? bytes : (size_t)mhc::kProbeSinkWords * 4, "dst");
  if (v.finish() != MHC_OK) return v.status();
  mhc::launch_bandwidth_probe((hipStream_t)stream, copy, (kind & MHC_PROBE_NONTEMPORAL) != 0, src, dst,
                              (int64_t)bytes);
  return launched("mhc_bandwidth_probe");
}

// ------------------------------------------------------------------ projection fwd
size_t mhc_proj_rms_h_workspace_size(int64_t tokens, int32_t n, int64_t C, mhc_dtype act) {
  if (tokens <= 0 || tokens > mhc::kMaxTokens || n < 1 || n > mhc::kMaxN || C <= 0 || C % 8 || C > mhc::kMaxC) return 0;
  return n == 4 ? mhc::proj_fwd_ws(tokens, C, act == MHC_F32)
                : mhc::gproj_fwd_ws(n, tokens, C, act == MHC_F32);
}

mhc_status mhc_proj_rms_h(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                          const void *X, const float *W, const float *alpha, const float *hbias,
                          float rms_eps, float *H_pre, float *H_post, float *H_res_logits,
                          float *saved, void *workspace, size_t workspace_bytes) {
  Validator v("mhc_proj_rms_h");
  v.dims(tokens, n, C, act);
  v.eps(rms_eps, "rms_eps");
  if (!v.ok()) return v.status();
  if (tokens == 0) return MHC_OK;
  const int64_t K = (int64_t)n * C;
  const int64_t J = (int64_t)n * n + 2 * n;
  v.in(X, tokens * K * esz(act), "X");
  v.in(W, K * J * 4, "W");
  v.in(alpha, 3 * 4, "alpha", true);
  v.in(hbias, J * 4, "hbias", true);
  v.out(H_pre, tokens * n * 4, "H_pre");
  v.out(H_post, tokens * n * 4, "H_post");
  v.out(H_res_logits, tokens * n * n * 4, "H_res_logits");
  v.out(saved, tokens * mhc::saved_stride(n) * 4, "saved", true);
  v.workspace(workspace, workspace_bytes,
              n == 4 ? mhc::proj_fwd_ws(tokens, C, act == MHC_F32)
                     : mhc::gproj_fwd_ws(n, tokens, C, act == MHC_F32));
  if (v.finish() != MHC_OK) return v.status();
  if (n == 4)
    mhc::launch_proj_fwd((hipStream_t)stream, act == MHC_F32, tokens, C, X, W, alpha, hbias, rms_eps,
                         H_pre, H_post, H_res_logits, saved, nullptr, 0, 0.f, workspace);
  else
    mhc::glaunch_proj_fwd((hipStream_t)stream, act == MHC_F32, n, tokens, C, X, W, alpha, hbias, rms_eps,
                          H_pre, H_post, H_res_logits, saved, nullptr, 0, 0.f, workspace);
  return launched("mhc_proj_rms_h");
}

mhc_status mhc_proj_rms_h_fma(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                              const void *X, const float *W, const float *alpha, const float *hbias,
                              float rms_eps, float *H_pre, float *H_post, float *H_res_logits,
                              float *saved, void *workspace, size_t workspace_bytes) {
  Validator v("mhc_proj_rms_h_fma");
  v.dims(tokens, n, C, act);
  v.eps(rms_eps, "rms_eps");
  if (v.ok() && (n != 4 || act != MHC_BF16)) v.fail(MHC_ERR_UNSUPPORTED, "the FMA form takes n == 4 and bf16 only");
  if (!v.ok()) return v.status();
  if (tokens == 0) return MHC_OK;
  const int64_t K = 4 * C;
  v.in(X, tokens * K * 2, "X");
  v.in(W, K * 24 * 4, "W");
  v.in(alpha, 3 * 4, "alpha", true);
  v.in(hbias, 24 * 4, "hbias", true);
  v.out(H_pre, tokens * 16, "H_pre");
  v.out(H_post, tokens * 16, "H_post");
  v.out(H_res_logits, tokens * 64, "H_res_logits");
  v.out(saved, tokens * mhc::kSavedStride * 4, "saved", true);
  v.workspace(workspace, workspace_bytes, mhc::proj_fwd_ws(tokens, C, false));
  if (v.finish() != MHC_OK) return v.status();
  mhc::launch_proj_fwd_fma((hipStream_t)stream, tokens, C, X, W, alpha, hbias, rms_eps, H_pre, H_post,
                           H_res_logits, saved, workspace);
  return launched("mhc_proj_rms_h_fma");
}

// ------------------------------------------------------------------ projection bwd
size_t mhc_proj_rms_h_bwd_workspace_size(int64_t tokens, int32_t n, int64_t C, mhc_dtype act) {
  if (tokens <= 0 || tokens > mhc::kMaxTokens || n < 1 || n > mhc::kMaxN || C <= 0 || C % 8 || C > mhc::kMaxC) return 0;
  return n == 4 ? mhc::proj_bwd_ws(tokens, C, act == MHC_F32)
                : mhc::gproj_bwd_ws(n, tokens, C, false, act == MHC_F32);
}

mhc_status mhc_proj_rms_h_bwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                              const void *X, const float *W, const float *alpha, const float *saved,
                              const float *H_pre, const float *H_post, const float *dH_pre,
                              const float *dH_post, const float *dH_res_logits, void *dX,
                              int32_t accumulate_dX, float *dW, float *dalpha, float *dhbias,
                              void *workspace, size_t workspace_bytes) {
  Validator v("mhc_proj_rms_h_bwd");
  v.dims(tokens, n, C, act);
  if (!v.ok()) return v.status();
  const int64_t K = (int64_t)n * C;
  const int64_t J = (int64_t)n * n + 2 * n;
  const hipStream_t s = (hipStream_t)stream;
  if (tokens == 0) {
    v.out(dW, K * J * 4, "dW", true);
    v.out(dalpha, 12, "dalpha", true);
    v.out(dhbias, J * 4, "dhbias", true);
    if (v.finish() != MHC_OK) return v.status();
    const bool any = zero_f32(s, dW, K * J) | zero_f32(s, dalpha, 3) | zero_f32(s, dhbias, J);
    return any ? launched("mhc_proj_rms_h_bwd") : MHC_OK;
  }
  v.in(X, tokens * K * esz(act), "X");
  v.in(W, K * J * 4, "W");
  v.in(alpha, 12, "alpha", true);
  v.in(saved, tokens * mhc::saved_stride(n) * 4, "saved");
  v.in(H_pre, tokens * n * 4, "H_pre");
  v.in(H_post, tokens * n * 4, "H_post");
  v.in(dH_pre, tokens * n * 4, "dH_pre");
  v.in(dH_post, tokens * n * 4, "dH_post");
  v.in(dH_res_logits, tokens * n * n * 4, "dH_res_logits");
  v.out(dX, tokens * K * esz(act), "dX");
  v.out(dW, K * J * 4, "dW", true);
  v.out(dalpha, 12, "dalpha", true);
  v.out(dhbias, J * 4, "dhbias", true);
  v.workspace(workspace, workspace_bytes,
              n == 4 ? mhc::proj_bwd_ws(tokens, C, act == MHC_F32)
                     : mhc::gproj_bwd_ws(n, tokens, C, false, act == MHC_F32));
  if (v.finish() != MHC_OK) return v.status();
  mhc::ProjBwdArgs a{};
  a.f32 = act == MHC_F32; a.N = tokens; a.C = C; a.X = X; a.W = W; a.alpha = alpha; a.saved = saved;
  a.H_pre = H_pre; a.H_post = H_post; a.dH_pre = dH_pre; a.dH_post = dH_post; a.dL = dH_res_logits;
  a.dH_res = nullptr; a.logits = nullptr; a.iters = 0; a.eps = 0.f; a.g = nullptr; a.dX = dX;
  a.accumulate = accumulate_dX != 0; a.dW = dW; a.dalpha = dalpha; a.dhbias = dhbias;
  a.dH_pre_out = nullptr; a.dL_out = nullptr; a.ws = workspace;
  if (n == 4)
    mhc::launch_proj_bwd(s, a);
  else
    mhc::glaunch_proj_bwd(s, n, a);
  return launched("mhc_proj_rms_h_bwd");
}

// ------------------------------------------------------------------ Sinkhorn
mhc_status mhc_sinkhorn_fwd(void *stream, int64_t count, int32_t n, const float *logits,
                            float *H_res, int32_t iters, float eps) {
  Validator v("mhc_sinkhorn_fwd");
  v.count(count);
  if (n <= 0) v.fail(MHC_ERR_SHAPE, "n must be > 0");
  else if (n > mhc::kMaxN) v.fail(MHC_ERR_UNSUPPORTED, "n must be <= 8");
  v.iters(iters);
  v.eps(eps, "eps");
  if (!v.ok()) return v.status();
  if (count == 0) return MHC_OK;
  v.in(logits, count * n * n * 4, "logits");
  v.out(H_res, count * n * n * 4, "H_res");
  if (v.finish() != MHC_OK) return v.status();
  if (n == 4)
    mhc::launch_sinkhorn_fwd((hipStream_t)stream, count, logits, H_res, iters, eps);
  else
    mhc::glaunch_sinkhorn_fwd((hipStream_t)stream, n, count, logits, H_res, iters, eps);
  return launched("mhc_sinkhorn_fwd");
}

mhc_status mhc_sinkhorn_bwd(void *stream, int64_t count, int32_t n, const float *dH_res,
                            const float *logits, float *dlogits, int32_t iters, float eps) {
  Validator v("mhc_sinkhorn_bwd");
  v.count(count);
  if (n <= 0) v.fail(MHC_ERR_SHAPE, "n must be > 0");
  else if (n > mhc::kMaxN) v.fail(MHC_ERR_UNSUPPORTED, "n must be <= 8");
  v.iters(iters);
  v.eps(eps, "eps");
  if (!v.ok()) return v.status();
  if (count == 0) return MHC_OK;
  v.in(dH_res, count * n * n * 4, "dH_res");
  v.in(logits, count * n * n * 4, "logits");
  v.out(dlogits, count * n * n * 4, "dlogits");
  if (v.finish() != MHC_OK) return v.status();
  if (n == 4)
    mhc::launch_sinkhorn_bwd((hipStream_t)stream, count, dH_res, logits, dlogits, iters, eps);
  else
    mhc::glaunch_sinkhorn_bwd((hipStream_t)stream, n, count, dH_res, logits, dlogits, iters, eps);
  return launched("mhc_sinkhorn_bwd");
}

// ------------------------------------------------------------------ h_aggregate
mhc_status mhc_h_aggregate_fwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                               const void *X, const float *H_pre, void *out) {
  Validator v("mhc_h_aggregate_fwd");
  v.dims(tokens, n, C, act);
  if (!v.ok()) return v.status();
  if (tokens == 0) return MHC_OK;
  v.in(X, tokens * n * C * esz(act), "X");
  v.in(H_pre, tokens * n * 4, "H_pre");
  v.out(out, tokens * C * esz(act), "out");
  if (v.finish() != MHC_OK) return v.status();
  if (n == 4)
    mhc::launch_h_aggregate_fwd((hipStream_t)stream, act == MHC_F32, tokens, C, X, H_pre, out);
  else
    mhc::glaunch_h_aggregate_fwd((hipStream_t)stream, act == MHC_F32, n, tokens, C, X, H_pre, out, n);
  return launched("mhc_h_aggregate_fwd");
}

mhc_status mhc_h_aggregate_bwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                               const void *g, const void *X, const float *H_pre, void *dX,
                               int32_t accumulate_dX, float *dH_pre) {
  Validator v("mhc_h_aggregate_bwd");
  v.dims(tokens, n, C, act);
  if (!v.ok()) return v.status();
  if (tokens == 0) return MHC_OK;
  v.in(g, tokens * C * esz(act), "g");
  v.in(X, tokens * n * C * esz(act), "X");
  v.in(H_pre, tokens * n * 4, "H_pre");
  v.out(dX, tokens * n * C * esz(act), "dX");
  v.out(dH_pre, tokens * n * 4, "dH_pre");
  if (v.finish() != MHC_OK) return v.status();
  if (n == 4)
    mhc::launch_h_aggregate_bwd((hipStream_t)stream, act == MHC_F32, tokens, C, g, X, H_pre, dX,
                                accumulate_dX != 0, dH_pre);
  else
    mhc::glaunch_h_aggregate_bwd((hipStream_t)stream, act == MHC_F32, n, tokens, C, g, X, H_pre, dX,
                                 accumulate_dX != 0, dH_pre);
  return launched("mhc_h_aggregate_bwd");
}

// ------------------------------------------------------------------ h_post_bda
mhc_status mhc_h_post_bda_fwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                              const void *X, const float *H_res, const float *H_post, const void *x,
                              const void *bias, void *out) {
  Validator v("mhc_h_post_bda_fwd");
  v.dims(tokens, n, C, act);
  if (!v.ok()) return v.status();
  if (tokens == 0) return MHC_OK;
  v.in(X, tokens * n * C * esz(act), "X");
  v.in(H_res, tokens * n * n * 4, "H_res");
  v.in(H_post, tokens * n * 4, "H_post");
  v.in(x, tokens * C * esz(act), "x");
  v.in(bias, C * esz(act), "bias", true);
  v.out(out, tokens * n * C * esz(act), "out");
  if (v.finish() != MHC_OK) return v.status();
  if (n == 4)
    mhc::launch_h_post_bda_fwd((hipStream_t)stream, act == MHC_F32, tokens, C, X, H_res, H_post, x, bias, out);
  else
    mhc::glaunch_h_post_bda_fwd((hipStream_t)stream, act == MHC_F32, n, tokens, C, X, H_res, H_post, x, bias, out);
  return launched("mhc_h_post_bda_fwd");
}

size_t mhc_h_post_bda_bwd_workspace_size(int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                                         int32_t with_dbias) {
  (void)act;
  if (tokens <= 0 || tokens > mhc::kMaxTokens || n < 1 || n > mhc::kMaxN || C <= 0 || C % 8 || C > mhc::kMaxC) return 0;
  return n == 4 ? mhc::h_post_bda_bwd_ws(tokens, C, with_dbias != 0) : mhc::gh_post_bda_bwd_ws(tokens, C, with_dbias != 0);
}

mhc_status mhc_h_post_bda_bwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                              const void *G, const void *X, const float *H_res,
                              const float *H_post, const void *x, const void *bias, void *dX,
                              float *dH_res, float *dH_post, void *dx, void *dbias,
                              void *workspace, size_t workspace_bytes) {
  Validator v("mhc_h_post_bda_bwd");
  v.dims(tokens, n, C, act);
  if (dbias && !bias) v.fail(MHC_ERR_ARG, "dbias requested without bias");
  if (!v.ok()) return v.status();
  const hipStream_t s = (hipStream_t)stream;
  if (tokens == 0) {
    v.out(dbias, C * esz(act), "dbias", true);
    if (v.finish() != MHC_OK) return v.status();
    return zero_act(s, dbias, C, act) ? launched("mhc_h_post_bda_bwd") : MHC_OK;
  }
  v.in(G, tokens * n * C * esz(act), "G");
  v.in(X, tokens * n * C * esz(act), "X");
  v.in(H_res, tokens * n * n * 4, "H_res");
  v.in(H_post, tokens * n * 4, "H_post");
  v.in(x, tokens * C * esz(act), "x");
  v.in(bias, C * esz(act), "bias", true);
  v.out(dX, tokens * n * C * esz(act), "dX", true);
  v.out(dH_res, tokens * n * n * 4, "dH_res");
  v.out(dH_post, tokens * n * 4, "dH_post");
  v.out(dx, tokens * C * esz(act), "dx");
  v.out(dbias, C * esz(act), "dbias", true);
  v.workspace(workspace, workspace_bytes, n == 4 ? mhc::h_post_bda_bwd_ws(tokens, C, dbias != nullptr) : mhc::gh_post_bda_bwd_ws(tokens, C, dbias != nullptr));
  if (v.finish() != MHC_OK) return v.status();
  if (n == 4)
    mhc::launch_h_post_bda_bwd(s, act == MHC_F32, tokens, C, G, X, H_res, H_post, x, bias, dX, dH_res,
                               dH_post, dx, dbias, workspace);
  else
    mhc::glaunch_h_post_bda_bwd(s, act == MHC_F32, n, tokens, C, G, X, H_res, H_post, x, bias, dX, dH_res,
                                dH_post, dx, dbias, workspace);
  return launched("mhc_h_post_bda_bwd");
}

// ------------------------------------------------------------------ stream mix / distribute
mhc_status mhc_stream_mix_fwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                              const void *X, const float *M, void *out) {
  Validator v("mhc_stream_mix_fwd");
  v.dims(tokens, n, C, act);
  if (!v.ok()) return v.status();
  if (tokens == 0) return MHC_OK;
  v.in(X, tokens * n * C * esz(act), "X");
  v.in(M, tokens * n * n * 4, "M");
  v.out(out, tokens * n * C * esz(act), "out");
  if (v.finish() != MHC_OK) return v.status();
  if (n == 4)
    mhc::launch_stream_mix_fwd((hipStream_t)stream, act == MHC_F32, tokens, C, X, M, out);
  else
    mhc::glaunch_stream_mix_fwd((hipStream_t)stream, act == MHC_F32, n, tokens, C, X, M, out);
  return launched("mhc_stream_mix_fwd");
}

mhc_status mhc_stream_mix_bwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                              const void *G, const void *X, const float *M, void *dX, float *dM) {
  Validator v("mhc_stream_mix_bwd");
  v.dims(tokens, n, C, act);
  if (!v.ok()) return v.status();
  if (tokens == 0) return MHC_OK;
  v.in(G, tokens * n * C * esz(act), "G");
  v.in(X, tokens * n * C * esz(act), "X");
  v.in(M, tokens * n * n * 4, "M");
  v.out(dX, tokens * n * C * esz(act), "dX");
  v.out(dM, tokens * n * n * 4, "dM");
  if (v.finish() != MHC_OK) return v.status();
  if (n == 4)
    mhc::launch_stream_mix_bwd((hipStream_t)stream, act == MHC_F32, tokens, C, G, X, M, dX, dM);
  else
    mhc::glaunch_stream_mix_bwd((hipStream_t)stream, act == MHC_F32, n, tokens, C, G, X, M, dX, dM);
  return launched("mhc_stream_mix_bwd");
}

mhc_status mhc_stream_distribute_fwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                                     const void *x, const float *H_post, void *out) {
  Validator v("mhc_stream_distribute_fwd");
  v.dims(tokens, n, C, act);
  if (!v.ok()) return v.status();
  if (tokens == 0) return MHC_OK;
  v.in(x, tokens * C * esz(act), "x");
  v.in(H_post, tokens * n * 4, "H_post");
  v.out(out, tokens * n * C * esz(act), "out");
  if (v.finish() != MHC_OK) return v.status();
  if (n == 4)
    mhc::launch_stream_distribute_fwd((hipStream_t)stream, act == MHC_F32, tokens, C, x, H_post, out);
  else
    mhc::glaunch_stream_distribute_fwd((hipStream_t)stream, act == MHC_F32, n, tokens, C, x, H_post, out);
  return launched("mhc_stream_distribute_fwd");
}

mhc_status mhc_stream_distribute_bwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                                     const void *G, const void *x, const float *H_post, void *dx,
                                     float *dH_post) {
  Validator v("mhc_stream_distribute_bwd");
  v.dims(tokens, n, C, act);
  if (!v.ok()) return v.status();
  if (tokens == 0) return MHC_OK;
  v.in(G, tokens * n * C * esz(act), "G");
  v.in(x, tokens * C * esz(act), "x");
  v.in(H_post, tokens * n * 4, "H_post");
  v.out(dx, tokens * C * esz(act), "dx");
  v.out(dH_post, tokens * n * 4, "dH_post");
  if (v.finish() != MHC_OK) return v.status();
  if (n == 4)
    mhc::launch_stream_distribute_bwd((hipStream_t)stream, act == MHC_F32, tokens, C, G, x, H_post, dx, dH_post);
  else
    mhc::glaunch_stream_distribute_bwd((hipStream_t)stream, act == MHC_F32, n, tokens, C, G, x, H_post, dx,
                                       dH_post);
  return launched("mhc_stream_distribute_bwd");
}

// ------------------------------------------------------------------ h_aggregate, one shared H_pre row
mhc_status mhc_h_aggregate_static_fwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                                      const void *X, const float *H_pre, void *out) {
  Validator v("mhc_h_aggregate_static_fwd");
  v.dims(tokens, n, C, act);
  if (!v.ok()) return v.status();
  if (tokens == 0) return MHC_OK;
  v.in(X, tokens * n * C * esz(act), "X");
  v.in(H_pre, n * 4, "H_pre");
  v.out(out, tokens * C * esz(act), "out");
  if (v.finish() != MHC_OK) return v.status();
  if (n == 4)
    mhc::launch_h_aggregate_fwd((hipStream_t)stream, act == MHC_F32, tokens, C, X, H_pre, out, 0);
  else
    mhc::glaunch_h_aggregate_fwd((hipStream_t)stream, act == MHC_F32, n, tokens, C, X, H_pre, out, 0);
  return launched("mhc_h_aggregate_static_fwd");
}

size_t mhc_h_aggregate_static_bwd_workspace_size(int64_t tokens, int32_t n, int64_t C, mhc_dtype act) {
  (void)act;
  if (tokens <= 0 || tokens > mhc::kMaxTokens || n < 1 || n > mhc::kMaxN || C <= 0 || C % 8 || C > mhc::kMaxC) return 0;
  return n == 4 ? mhc::h_aggregate_static_bwd_ws(tokens) : mhc::gh_aggregate_static_bwd_ws(n, tokens);
}

mhc_status mhc_h_aggregate_static_bwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                                      const void *g, const void *X, const float *H_pre, void *dX,
                                      int32_t accumulate_dX, float *dH_pre, void *workspace,
                                      size_t workspace_bytes) {
  Validator v("mhc_h_aggregate_static_bwd");
  v.dims(tokens, n, C, act);
  if (!v.ok()) return v.status();
  const hipStream_t s = (hipStream_t)stream;
  if (tokens == 0) {
    v.out(dH_pre, n * 4, "dH_pre");
    if (v.finish() != MHC_OK) return v.status();
    return zero_f32(s, dH_pre, n) ? launched("mhc_h_aggregate_static_bwd") : MHC_OK;
  }
  v.in(g, tokens * C * esz(act), "g");
  v.in(X, tokens * n * C * esz(act), "X");
  v.in(H_pre, n * 4, "H_pre");
  v.out(dX, tokens * n * C * esz(act), "dX");
  v.out(dH_pre, n * 4, "dH_pre");
  v.workspace(workspace, workspace_bytes, n == 4 ? mhc::h_aggregate_static_bwd_ws(tokens) : mhc::gh_aggregate_static_bwd_ws(n, tokens));
  if (v.finish() != MHC_OK) return v.status();
  if (n == 4)
    mhc::launch_h_aggregate_static_bwd(s, act == MHC_F32, tokens, C, g, X, H_pre, dX, accumulate_dX != 0,
                                       dH_pre, workspace);
  else
    mhc::glaunch_h_aggregate_static_bwd(s, act == MHC_F32, n, tokens, C, g, X, H_pre, dX, accumulate_dX != 0,
                                        dH_pre, workspace);
  return launched("mhc_h_aggregate_static_bwd");
}

// ------------------------------------------------------------------ fused pre pass
size_t mhc_pre_fwd_workspace_size(int64_t tokens, int32_t n, int64_t C, mhc_dtype act) {
  return mhc_proj_rms_h_workspace_size(tokens, n, C, act);
}

mhc_status mhc_pre_fwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                       const void *X, const float *W, const float *alpha, const float *hbias,
                       float rms_eps, int32_t iters, float eps, float *H_pre, float *H_post,
                       float *H_res, float *H_res_logits, float *saved, void *agg,
                       void *workspace, size_t workspace_bytes) {
  Validator v("mhc_pre_fwd");
  if (!pre_fwd_check(v, tokens, n, C, act, X, W, alpha, hbias, rms_eps, iters, eps, H_pre, H_post, H_res,
                     H_res_logits, saved, agg))
    return v.status();
  if (tokens == 0) return MHC_OK;
  v.workspace(workspace, workspace_bytes, pre_fwd_ws(tokens, n, C, act));
  if (v.finish() != MHC_OK) return v.status();
  pre_fwd_launch((hipStream_t)stream, tokens, n, C, act, X, W, alpha, hbias, rms_eps, iters, eps, H_pre, H_post,
                 H_res, H_res_logits, saved, agg, workspace);
  return launched("mhc_pre_fwd");
}

mhc_status mhc_pre_fwd_noalloc(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                               const void *X, const float *W, const float *alpha, const float *hbias,
                               float rms_eps, int32_t iters, float eps, float *H_pre, float *H_post,
                               float *H_res, float *H_res_logits, float *saved, void *agg) {
  Validator v("mhc_pre_fwd_noalloc");
  if (!pre_fwd_check(v, tokens, n, C, act, X, W, alpha, hbias, rms_eps, iters, eps, H_pre, H_post, H_res,
                     H_res_logits, saved, agg))
    return v.status();
  if (tokens == 0) return MHC_OK;
  const size_t need = pre_fwd_ws(tokens, n, C, act);
  if (need > (size_t)MHC_NOALLOC_SCRATCH_BYTES)
    v.fail(MHC_ERR_UNSUPPORTED, "this call needs " + std::to_string(need) +
                                    " bytes of scratch; the static scratch holds " +
                                    std::to_string((size_t)MHC_NOALLOC_SCRATCH_BYTES) +
                                    " (use mhc_pre_fwd with a workspace)");
  if (v.finish() != MHC_OK) return v.status();
  void *ws = nullptr;
  const mhc_status st = scratch_of_current_device(&ws, "mhc_pre_fwd_noalloc");
  if (st != MHC_OK) return st;
  pre_fwd_launch((hipStream_t)stream, tokens, n, C, act, X, W, alpha, hbias, rms_eps, iters, eps, H_pre, H_post,
                 H_res, H_res_logits, saved, agg, ws);
  return launched("mhc_pre_fwd_noalloc");
}

// ------------------------------------------------------------------ RMSNorm of the aggregated stream
mhc_status mhc_rmsnorm_fwd(void *stream, int64_t tokens, int64_t C, mhc_dtype act, const void *x,
                           const float *gamma, float eps, void *y) {
  Validator v("mhc_rmsnorm_fwd");
  v.rows(tokens, C, act);
  v.eps(eps, "eps");
  if (!v.ok()) return v.status();
  if (tokens == 0) return MHC_OK;
  v.in(x, tokens * C * esz(act), "x");
  v.in(gamma, C * 4, "gamma", true);
  v.out(y, tokens * C * esz(act), "y");
  if (v.finish() != MHC_OK) return v.status();
  mhc::launch_rmsnorm_fwd((hipStream_t)stream, act == MHC_F32, tokens, C, x, gamma, eps, y);
  return launched("mhc_rmsnorm_fwd");
}

size_t mhc_rmsnorm_bwd_workspace_size(int64_t tokens, int64_t C, mhc_dtype act, int32_t with_dgamma) {
  (void)act;
  if (tokens <= 0 || tokens > mhc::kMaxTokens || C <= 0 || C % 8 || C > mhc::kMaxC) return 0;
  return mhc::rmsnorm_bwd_ws(tokens, C, with_dgamma != 0);
}

mhc_status mhc_rmsnorm_bwd(void *stream, int64_t tokens, int64_t C, mhc_dtype act, const void *dy,
                           const void *x, const float *gamma, float eps, void *dx,
                           int32_t accumulate_dx, float *dgamma, void *workspace,
                           size_t workspace_bytes) {
  Validator v("mhc_rmsnorm_bwd");
  v.rows(tokens, C, act);
  v.eps(eps, "eps");
  if (!v.ok()) return v.status();
  const hipStream_t s = (hipStream_t)stream;
  if (tokens == 0) {
    v.out(dgamma, C * 4, "dgamma", true);
    if (v.finish() != MHC_OK) return v.status();
    return zero_f32(s, dgamma, C) ? launched("mhc_rmsnorm_bwd") : MHC_OK;
  }
  v.in(dy, tokens * C * esz(act), "dy");
  v.in(x, tokens * C * esz(act), "x");
  v.in(gamma, C * 4, "gamma", true);
  v.out(dx, tokens * C * esz(act), "dx");
  v.out(dgamma, C * 4, "dgamma", true);
  v.workspace(workspace, workspace_bytes, mhc::rmsnorm_bwd_ws(tokens, C, dgamma != nullptr));
  if (v.finish() != MHC_OK) return v.status();
  mhc::launch_rmsnorm_bwd(s, act == MHC_F32, tokens, C, dy, x, gamma, eps, dx, accumulate_dx != 0, dgamma,
                          workspace);
  return launched("mhc_rmsnorm_bwd");
}

mhc_status mhc_pre_rmsnorm_fwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                               const void *X, const float *W, const float *alpha, const float *hbias,
                               float rms_eps, int32_t iters, float eps, const float *gamma,
                               float norm_eps, float *H_pre, float *H_post, float *H_res,
                               float *H_res_logits, float *saved, void *agg, void *normed,
                               void *workspace, size_t workspace_bytes) {
  Validator v("mhc_pre_rmsnorm_fwd");
  v.dims(tokens, n, C, act);
  v.eps(rms_eps, "rms_eps");
  v.eps(eps, "eps");
  v.eps(norm_eps, "norm_eps");
  v.iters(iters);
  if (!v.ok()) return v.status();
  if (tokens == 0) return MHC_OK;
  const int64_t K = (int64_t)n * C;
  const int64_t J = (int64_t)n * n + 2 * n;
  v.in(X, tokens * K * esz(act), "X");
  v.in(W, K * J * 4, "W");
  v.in(alpha, 12, "alpha", true);
  v.in(hbias, J * 4, "hbias", true);
  v.in(gamma, C * 4, "gamma", true);
  v.out(H_pre, tokens * n * 4, "H_pre");
  v.out(H_post, tokens * n * 4, "H_post");
  v.out(H_res, tokens * n * n * 4, "H_res");
  v.out(H_res_logits, tokens * n * n * 4, "H_res_logits");
  v.out(saved, tokens * mhc::saved_stride(n) * 4, "saved", true);
  v.out(agg, tokens * C * esz(act), "agg");
  v.out(normed, tokens * C * esz(act), "normed");
  v.workspace(workspace, workspace_bytes,
              n == 4 ? mhc::proj_fwd_ws(tokens, C, act == MHC_F32)
                     : mhc::gproj_fwd_ws(n, tokens, C, act == MHC_F32));
  if (v.finish() != MHC_OK) return v.status();
  const hipStream_t s = (hipStream_t)stream;
  if (n == 4) {
    mhc::launch_proj_fwd(s, act == MHC_F32, tokens, C, X, W, alpha, hbias, rms_eps, H_pre, H_post,
                         H_res_logits, saved, H_res, iters, eps, workspace);
    mhc::launch_h_aggregate_rmsnorm_fwd(s, act == MHC_F32, tokens, C, X, H_pre, gamma, norm_eps, agg, normed);
  } else {  // other n: aggregate, then the norm of the stored agg (same result, one more pass over agg)
    mhc::glaunch_proj_fwd(s, act == MHC_F32, n, tokens, C, X, W, alpha, hbias, rms_eps, H_pre, H_post,
                          H_res_logits, saved, H_res, iters, eps, workspace);
    mhc::glaunch_h_aggregate_fwd(s, act == MHC_F32, n, tokens, C, X, H_pre, agg, n);
    mhc::launch_rmsnorm_fwd(s, act == MHC_F32, tokens, C, agg, gamma, norm_eps, normed);
  }
  return launched("mhc_pre_rmsnorm_fwd");
}

// ------------------------------------------------------------------ fused pre backward with the norm
namespace {
struct PreNormBwdWs {
  size_t pre, dagg, norm, total;
};
PreNormBwdWs pre_norm_bwd_ws(int64_t tokens, int32_t n, int64_t C, mhc_dtype act, bool dgamma) {
  auto a256 = [](size_t b) { return (b + 255) / 256 * 256; };
  PreNormBwdWs w{};
  w.pre = a256(n == 4 ? mhc::proj_bwd_ws(tokens, C, act == MHC_F32)
                      : mhc::gproj_bwd_ws(n, tokens, C, true, act == MHC_F32));
  w.dagg = a256((size_t)tokens * C * esz(act));
  w.norm = a256(mhc::rmsnorm_bwd_ws(tokens, C, dgamma));
  w.total = w.pre + w.dagg + w.norm;
  return w;
}
}  // namespace

size_t mhc_pre_rmsnorm_bwd_workspace_size(int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                                          int32_t with_dgamma) {
  if (tokens <= 0 || tokens > mhc::kMaxTokens || n < 1 || n > mhc::kMaxN || C <= 0 || C % 8 || C > mhc::kMaxC)
    return 0;
  return pre_norm_bwd_ws(tokens, n, C, act, with_dgamma != 0).total;
}

mhc_status mhc_pre_rmsnorm_bwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                               const void *dy, const void *agg, const float *gamma, float norm_eps,
                               const void *g_fork, const float *dH_post, const float *dH_res, const void *X,
                               const float *W, const float *alpha, const float *saved, const float *H_pre,
                               const float *H_post, const float *H_res_logits, int32_t iters, float eps,
                               const void *post_G, const float *post_H_res, void *dX, int32_t accumulate_dX,
                               float *dW, float *dalpha, float *dhbias, float *dgamma, void *d_agg_out,
                               void *workspace, size_t workspace_bytes) {
  Validator v("mhc_pre_rmsnorm_bwd");
  v.dims(tokens, n, C, act);
  v.eps(eps, "eps");
  v.eps(norm_eps, "norm_eps");
  v.iters(iters);
  if ((post_G == nullptr) != (post_H_res == nullptr))
    v.fail(MHC_ERR_ARG, "post_G and post_H_res must be given together");
  if (!v.ok()) return v.status();
  const int64_t K = (int64_t)n * C;
  const int64_t J = (int64_t)n * n + 2 * n;
  const hipStream_t s = (hipStream_t)stream;
  if (tokens == 0) {
    v.out(dW, K * J * 4, "dW", true);
    v.out(dalpha, 12, "dalpha", true);
    v.out(dhbias, J * 4, "dhbias", true);
    v.out(dgamma, C * 4, "dgamma", true);
    if (v.finish() != MHC_OK) return v.status();
    const bool any = zero_f32(s, dW, K * J) | zero_f32(s, dalpha, 3) | zero_f32(s, dhbias, J) | zero_f32(s, dgamma, C);
    return any ? launched("mhc_pre_rmsnorm_bwd") : MHC_OK;
  }
  v.in(dy, tokens * C * esz(act), "dy");
  v.in(agg, tokens * C * esz(act), "agg");
  v.in(gamma, C * 4, "gamma", true);
  v.in(g_fork, tokens * C * esz(act), "g_fork", true);
  v.in(dH_post, tokens * n * 4, "dH_post");
  v.in(dH_res, tokens * n * n * 4, "dH_res");
  v.in(X, tokens * K * esz(act), "X");
  v.in(W, K * J * 4, "W");
  v.in(alpha, 12, "alpha", true);
  v.in(saved, tokens * mhc::saved_stride(n) * 4, "saved");
  v.in(H_pre, tokens * n * 4, "H_pre");
  v.in(H_post, tokens * n * 4, "H_post");
  v.in(H_res_logits, tokens * n * n * 4, "H_res_logits");
  v.in(post_G, tokens * K * esz(act), "post_G", true);
  v.in(post_H_res, tokens * n * n * 4, "post_H_res", true);
  v.out(dX, tokens * K * esz(act), "dX");
  v.out(dW, K * J * 4, "dW", true);
  v.out(dalpha, 12, "dalpha", true);
  v.out(dhbias, J * 4, "dhbias", true);
  v.out(dgamma, C * 4, "dgamma", true);
  v.out(d_agg_out, tokens * C * esz(act), "d_agg_out", true);
  const PreNormBwdWs lay = pre_norm_bwd_ws(tokens, n, C, act, dgamma != nullptr);
  v.workspace(workspace, workspace_bytes, lay.total);
  if (v.finish() != MHC_OK) return v.status();
  char *ws = (char *)workspace;
  void *dagg = d_agg_out ? d_agg_out : (void *)(ws + lay.pre);
  void *norm_ws = ws + lay.pre + lay.dagg;
  mhc::ProjBwdArgs a{};
  a.f32 = act == MHC_F32; a.N = tokens; a.C = C; a.X = X; a.W = W; a.alpha = alpha; a.saved = saved;
  a.H_pre = H_pre; a.H_post = H_post; a.dH_pre = nullptr; a.dH_post = dH_post; a.dL = nullptr;
  a.dH_res = dH_res; a.logits = H_res_logits; a.iters = iters; a.eps = eps; a.g = dagg; a.dX = dX;
  a.accumulate = accumulate_dX != 0; a.dW = dW; a.dalpha = dalpha; a.dhbias = dhbias;
  a.dH_pre_out = nullptr; a.dL_out = nullptr; a.ws = ws;
  a.post_G = post_G; a.post_H_res = post_H_res;
  // The norm's backward into d_agg (agg's own gradient as the accumulation base), then the pre
  // backward on it.  A single pass forming d_agg and dH_pre together (so d_agg is read once less)
  // measured slower at 16384 x 7168: holding the norm's rows and X's together takes 150-208 VGPRs,
  // one workgroup per CU, where the separate dH_pre pass keeps several per CU.
  if (g_fork) copy16(s, g_fork, dagg, tokens * C * (int64_t)esz(act));
  mhc::launch_rmsnorm_bwd(s, act == MHC_F32, tokens, C, dy, agg, gamma, norm_eps, dagg, g_fork != nullptr, dgamma,
                          norm_ws);
  if (n == 4)
    mhc::launch_proj_bwd(s, a);
  else
    mhc::glaunch_proj_bwd(s, n, a);
  return launched("mhc_pre_rmsnorm_bwd");
}

size_t mhc_pre_bwd_workspace_size(int64_t tokens, int32_t n, int64_t C, mhc_dtype act) {
  if (tokens <= 0 || tokens > mhc::kMaxTokens || n < 1 || n > mhc::kMaxN || C <= 0 || C % 8 || C > mhc::kMaxC) return 0;
  return n == 4 ? mhc::proj_bwd_ws(tokens, C, act == MHC_F32)
                : mhc::gproj_bwd_ws(n, tokens, C, true, act == MHC_F32);
}

mhc_status mhc_pre_bwd(void *stream, int64_t tokens, int32_t n, int64_t C, mhc_dtype act,
                       const void *g, const float *dH_post, const float *dH_res, const void *X,
                       const float *W, const float *alpha, const float *saved, const float *H_pre,
                       const float *H_post, const float *H_res_logits, int32_t iters, float eps,
                       const void *post_G, const float *post_H_res, void *dX,
                       int32_t accumulate_dX, float *dW, float *dalpha, float *dhbias,
                       float *dH_pre_out, float *dlogits_out, void *workspace,
                       size_t workspace_bytes) {
  Validator v("mhc_pre_bwd");
  v.dims(tokens, n, C, act);
  v.eps(eps, "eps");
  v.iters(iters);
  if ((post_G == nullptr) != (post_H_res == nullptr))
    v.fail(MHC_ERR_ARG, "post_G and post_H_res must be given together");
  if (!v.ok()) return v.status();
  const int64_t K = (int64_t)n * C;
  const int64_t J = (int64_t)n * n + 2 * n;
  const hipStream_t s = (hipStream_t)stream;
  if (tokens == 0) {
    v.out(dW, K * J * 4, "dW", true);
    v.out(dalpha, 12, "dalpha", true);
    v.out(dhbias, J * 4, "dhbias", true);
    if (v.finish() != MHC_OK) return v.status();
    const bool any = zero_f32(s, dW, K * J) | zero_f32(s, dalpha, 3) | zero_f32(s, dhbias, J);
    return any ? launched("mhc_pre_bwd") : MHC_OK;
  }
  v.in(g, tokens * C * esz(act), "g");
  v.in(dH_post, tokens * n * 4, "dH_post");
  v.in(dH_res, tokens * n * n * 4, "dH_res");
  v.in(X, tokens * K * esz(act), "X");
  v.in(W, K * J * 4, "W");
  v.in(alpha, 12, "alpha", true);
  v.in(saved, tokens * mhc::saved_stride(n) * 4, "saved");
  v.in(H_pre, tokens * n * 4, "H_pre");
  v.in(H_post, tokens * n * 4, "H_post");
  v.in(H_res_logits, tokens * n * n * 4, "H_res_logits");
  v.in(post_G, tokens * K * esz(act), "post_G", true);
  v.in(post_H_res, tokens * n * n * 4, "post_H_res", true);
  v.out(dX, tokens * K * esz(act), "dX");
  v.out(dW, K * J * 4, "dW", true);
  v.out(dalpha, 12, "dalpha", true);
  v.out(dhbias, J * 4, "dhbias", true);
  v.out(dH_pre_out, tokens * n * 4, "dH_pre_out", true);
  v.out(dlogits_out, tokens * n * n * 4, "dlogits_out", true);
  v.workspace(workspace, workspace_bytes,
              n == 4 ? mhc::proj_bwd_ws(tokens, C, act == MHC_F32)
                     : mhc::gproj_bwd_ws(n, tokens, C, true, act == MHC_F32));
  if (v.finish() != MHC_OK) return v.status();
  mhc::ProjBwdArgs a{};
  a.f32 = act == MHC_F32; a.N = tokens; a.C = C; a.X = X; a.W = W; a.alpha = alpha; a.saved = saved;
  a.H_pre = H_pre; a.H_post = H_post; a.dH_pre = nullptr; a.dH_post = dH_post; a.dL = nullptr;
  a.dH_res = dH_res; a.logits = H_res_logits; a.iters = iters; a.eps = eps; a.g = g; a.dX = dX;
  a.accumulate = accumulate_dX != 0; a.dW = dW; a.dalpha = dalpha; a.dhbias = dhbias;
  a.dH_pre_out = dH_pre_out; a.dL_out = dlogits_out; a.ws = workspace;
  a.post_G = post_G; a.post_H_res = post_H_res;
  if (n == 4)
    mhc::launch_proj_bwd(s, a);
  else
    mhc::glaunch_proj_bwd(s, n, a);
  return launched("mhc_pre_bwd");
}

}  // extern "C"
