// C ABI of the S2-Attn library: argument checks, workspace layout and kernel
// dispatch.  Every entry point validates all arguments before enqueuing any
// GPU work and never lets an exception escape.
#include "s2attn.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <exception>
#include <mutex>
#include <string>

#include "kernels.hpp"
#include "lora_kernels.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(S2ATTN_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Test hook for the HIP-error status path: when S2ATTN_TEST_HIP_ERROR names
// a nonzero hipError_t code, every call that has passed its argument checks
// fails with S2ATTN_EHIP before making any HIP call, as a failed launch would.
int injected_hip_error() {
  const char* v = std::getenv("S2ATTN_TEST_HIP_ERROR");
  if (v == nullptr || *v == '\0') return S2ATTN_OK;
  const long code = std::strtol(v, nullptr, 10);
  if (code == 0) return S2ATTN_OK;
  return fail(S2ATTN_EHIP, "HIP error " + std::to_string(code) + " (injected by S2ATTN_TEST_HIP_ERROR)");
}

template <class F>
int guarded(F&& f) {
  try {
    return f();
  } catch (const std::exception& e) {
    return fail(S2ATTN_EHIP, std::string("internal error: ") + e.what());
  } catch (...) {
    return fail(S2ATTN_EHIP, "internal error");
  }
}

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Shape rules.  Returns S2ATTN_OK or an error status (message recorded).
int check_shape(int B, int N, int H, int Hkv, int D, int G, int shift, int pattern = S2ATTN_HEADS_SECOND_HALF) {
  if (B < 0 || N < 0) return fail(S2ATTN_EINVAL, "B and N must be >= 0");
  if (H < 1 || Hkv < 1) return fail(S2ATTN_EINVAL, "H and Hkv must be >= 1");
  if (H % Hkv != 0) return fail(S2ATTN_EINVAL, "H must be a multiple of Hkv");
  if (G < 1) return fail(S2ATTN_EINVAL, "G must be >= 1");
  if (N % G != 0) return fail(S2ATTN_EINVAL, "N must be a multiple of G");
  if (shift < 0 || shift >= G) return fail(S2ATTN_EINVAL, "shift must lie in [0, G)");
  if (pattern != S2ATTN_HEADS_SECOND_HALF && pattern != S2ATTN_HEADS_ALTERNATE)
    return fail(S2ATTN_EINVAL, "head_pattern must be S2ATTN_HEADS_SECOND_HALF or S2ATTN_HEADS_ALTERNATE");
  if (pattern == S2ATTN_HEADS_SECOND_HALF && shift > 0 && (H % 2 != 0 || Hkv % 2 != 0))
    return fail(S2ATTN_EINVAL, "with shift > 0, H and Hkv must be even (heads split in halves)");
  if (D < 1) return fail(S2ATTN_EINVAL, "D must be >= 1");
  if (D != 64 && D != 128) return fail(S2ATTN_EUNSUPPORTED, "D must be 64 or 128");
  // Element counts in 64-bit; workgroup counts must fit a 1-D grid.
  const double elems = (double)B * N * H * D;
  if (elems > 4.0e18) return fail(S2ATTN_EINVAL, "tensor too large");
  // Kernels address a tile of 64 consecutive rows with 32-bit offsets.
  if (64.0 * H * D >= 2147483648.0) return fail(S2ATTN_EINVAL, "H * D too large");
  const double wgs = (double)B * H * ((double)N / G) * ((G + 31) / 32);
  if (wgs > 2147483647.0) return fail(S2ATTN_EINVAL, "too many work items for one launch");
  return S2ATTN_OK;
}

struct Buf {
  const void* p;
  size_t bytes;
  const char* name;
};

bool overlap(const Buf& a, const Buf& b) {
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Null/alignment checks on all buffers and no overlap between any output and
// any other buffer.
int check_buffers(const Buf* in, int n_in, const Buf* out, int n_out) {
  for (int i = 0; i < n_in + n_out; ++i) {
    const Buf& b = i < n_in ? in[i] : out[i - n_in];
    if (b.p == nullptr) return fail(S2ATTN_EINVAL, std::string(b.name) + " is NULL");
    if (((uintptr_t)b.p & 15u) != 0) return fail(S2ATTN_EINVAL, std::string(b.name) + " is not 16-byte aligned");
  }
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlap(out[i], in[j]))
        return fail(S2ATTN_EINVAL, std::string(out[i].name) + " overlaps " + in[j].name);
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(out[i], out[j]))
        return fail(S2ATTN_EINVAL, std::string(out[i].name) + " overlaps " + out[j].name);
  }
  return S2ATTN_OK;
}

int check_rope(double base, double pos_scale) {
  if (!std::isfinite(base) || !(base > 0.0)) return fail(S2ATTN_EINVAL, "rope_base must be finite and > 0");
  if (!std::isfinite(pos_scale) || !(pos_scale > 0.0))
    return fail(S2ATTN_EINVAL, "pos_scale must be finite and > 0");
  return S2ATTN_OK;
}

s2a::RopeTable make_rope(int D, double base, double pos_scale) {
  s2a::RopeTable t{};
  const double two_pi = 6.283185307179586;
  for (int i = 0; i < D / 2; ++i) t.rev[i] = std::pow(base, -2.0 * i / D) / (pos_scale * two_pi);
  return t;
}

s2a::Shape make_shape(int B, int N, int H, int Hkv, int D, int G, int shift, int pattern) {
  return s2a::Shape{B, N, H, Hkv, D, G, shift, G > 0 ? N / G : 0, pattern};
}

size_t q_bytes(int B, int N, int H, int D) { return (size_t)B * N * H * D * 2; }
size_t stat_bytes(int B, int N, int H) { return (size_t)B * H * N * 4; }

int do_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int N, int H, int Hkv,
           int D, int G, int shift, const double* rope, void* ws, size_t ws_bytes, void* stream,
           int pattern = S2ATTN_HEADS_SECOND_HALF) {
  int st = check_shape(B, N, H, Hkv, D, G, shift, pattern);
  if (st) return st;
  if (rope && (st = check_rope(rope[0], rope[1]))) return st;
  if (B == 0 || N == 0) return S2ATTN_OK;
  const size_t qb = q_bytes(B, N, H, D), kb = q_bytes(B, N, Hkv, D);
  Buf in[3] = {{q, qb, "q"}, {k, kb, "k"}, {v, kb, "v"}};
  Buf outs[3] = {{out, qb, "out"}, {nullptr, 0, ""}, {nullptr, 0, ""}};
  int n_out = 1;
  if (lse) outs[n_out++] = Buf{lse, stat_bytes(B, N, H), "lse"};
  if (rope) outs[n_out++] = Buf{ws, round_up(kb), "workspace"};
  st = check_buffers(in, 3, outs, n_out);
  if (st) return st;
  if (rope && ws_bytes < round_up(kb)) return fail(S2ATTN_EINVAL, "workspace too small");
  if (rope && ((uintptr_t)ws & (kAlign - 1)) != 0) return fail(S2ATTN_EINVAL, "workspace is not 256-byte aligned");
  if ((st = injected_hip_error())) return st;
  const hipStream_t s = (hipStream_t)stream;
  s2a::FwdArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.out = (uint16_t*)out;
  a.lse = lse;
  a.s = make_shape(B, N, H, Hkv, D, G, shift, pattern);
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
  hipError_t e;
  if (rope) {
    const s2a::RopeTable t = make_rope(D, rope[0], rope[1]);
    uint16_t* krot = (uint16_t*)ws;
    if ((e = s2a::launch_rope_rotate(a.k, krot, a.s, Hkv, t, 1.f, s)) != hipSuccess) return hip_fail(e, "rope(k)");
    a.k = krot;
    if ((e = s2a::launch_fwd(a, &t, s)) != hipSuccess) return hip_fail(e, "forward");
  } else {
    if ((e = s2a::launch_fwd(a, nullptr, s)) != hipSuccess) return hip_fail(e, "forward");
  }
  return S2ATTN_OK;
}

int do_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse, const void* dout,
           void* dq, void* dk, void* dv, int B, int N, int H, int Hkv, int D, int G, int shift, const double* rope,
           void* ws, size_t ws_bytes, void* stream, int pattern = S2ATTN_HEADS_SECOND_HALF) {
  int st = check_shape(B, N, H, Hkv, D, G, shift, pattern);
  if (st) return st;
  if (rope && (st = check_rope(rope[0], rope[1]))) return st;
  if (B == 0 || N == 0) return S2ATTN_OK;
  const size_t qb = q_bytes(B, N, H, D), kb = q_bytes(B, N, Hkv, D), sb = stat_bytes(B, N, H);
  const size_t stats = 2 * round_up(sb);  // -Delta, then -lse*log2(e)
  // with RoPE, then the rotated and scaled q copy and the rotated k copy
  const size_t need = stats + (rope ? round_up(qb) + round_up(kb) : 0);
  Buf in[6] = {{q, qb, "q"}, {k, kb, "k"}, {v, kb, "v"}, {out, qb, "out"}, {lse, sb, "lse"}, {dout, qb, "dout"}};
  Buf outs[4] = {{dq, qb, "dq"}, {dk, kb, "dk"}, {dv, kb, "dv"}, {ws, need, "workspace"}};
  st = check_buffers(in, 6, outs, 4);
  if (st) return st;
  if (ws_bytes < need) return fail(S2ATTN_EINVAL, "workspace too small");
  if (((uintptr_t)ws & (kAlign - 1)) != 0) return fail(S2ATTN_EINVAL, "workspace is not 256-byte aligned");
  if ((st = injected_hip_error())) return st;
  const hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  float* ndelta = (float*)w;
  float* nlse2 = (float*)(w + round_up(sb));
  s2a::BwdArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.dout = (const uint16_t*)dout;
  a.nlse2 = nlse2;
  a.ndelta = ndelta;
  a.dq = (uint16_t*)dq;
  a.dk = (uint16_t*)dk;
  a.dv = (uint16_t*)dv;
  a.s = make_shape(B, N, H, Hkv, D, G, shift, pattern);
  a.scale = (float)(1.0 / std::sqrt((double)D));
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
  hipError_t e;
  s2a::RopeTable t{};
  if (rope) {
    // Rotated operands, rotated once here rather than once per reuse (each
    // q row is read by every k/v tile of its group): q as the logit operand
    // bf16(rotated q * log2(e)/sqrt(D)), k as bf16(rotated k).
    t = make_rope(D, rope[0], rope[1]);
    uint16_t* qs = (uint16_t*)(w + stats);
    uint16_t* krot = (uint16_t*)(w + stats + round_up(qb));
    if ((e = s2a::launch_rope_rotate(a.q, qs, a.s, H, t, a.scale_log2, s)) != hipSuccess)
      return hip_fail(e, "rope(q)");
    if ((e = s2a::launch_rope_rotate(a.k, krot, a.s, Hkv, t, 1.f, s)) != hipSuccess) return hip_fail(e, "rope(k)");
    a.q = qs;
    a.k = krot;
  }
  if ((e = s2a::launch_bwd_delta((const uint16_t*)out, (const uint16_t*)dout, lse, ndelta, nlse2, a.s, s)) !=
      hipSuccess)
    return hip_fail(e, "backward preprocess");
  if ((e = s2a::launch_bwd_dkdv(a, rope ? &t : nullptr, s)) != hipSuccess) return hip_fail(e, "backward dk/dv");
  if ((e = s2a::launch_bwd_dq(a, rope ? &t : nullptr, s)) != hipSuccess) return hip_fail(e, "backward dq");
  return S2ATTN_OK;
}

// Stage entry points of the backward (no RoPE).
enum class Stage { kPre, kDkdv, kDq };

int do_bwd_stage(Stage stage, const void* q, const void* k, const void* v, const void* out, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, int B, int N, int H, int Hkv, int D, int G,
                 int shift, const void* ws, size_t ws_bytes, void* stream) {
  const int pattern = S2ATTN_HEADS_SECOND_HALF;
  int st = check_shape(B, N, H, Hkv, D, G, shift);
  if (st) return st;
  if (B == 0 || N == 0) return S2ATTN_OK;
  const size_t qb = q_bytes(B, N, H, D), kb = q_bytes(B, N, Hkv, D), sb = stat_bytes(B, N, H);
  const size_t need = 2 * round_up(sb);  // -Delta, -lse*log2(e)
  if (ws_bytes < need) return fail(S2ATTN_EINVAL, "workspace too small");
  if (ws == nullptr || ((uintptr_t)ws & (kAlign - 1)) != 0)
    return fail(S2ATTN_EINVAL, "workspace is NULL or not 256-byte aligned");
  const hipStream_t s = (hipStream_t)stream;
  float* ndelta = (float*)ws;
  float* nlse2 = (float*)((char*)ws + round_up(sb));
  s2a::BwdArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.dout = (const uint16_t*)dout;
  a.nlse2 = nlse2;
  a.ndelta = ndelta;
  a.dq = (uint16_t*)dq;
  a.dk = (uint16_t*)dk;
  a.dv = (uint16_t*)dv;
  a.s = make_shape(B, N, H, Hkv, D, G, shift, pattern);
  a.scale = (float)(1.0 / std::sqrt((double)D));
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
  hipError_t e = hipSuccess;
  if (stage == Stage::kPre) {
    Buf in[3] = {{out, qb, "out"}, {dout, qb, "dout"}, {lse, sb, "lse"}};
    Buf outs[1] = {{ws, need, "workspace"}};
    if ((st = check_buffers(in, 3, outs, 1))) return st;
    if ((st = injected_hip_error())) return st;
    e = s2a::launch_bwd_delta((const uint16_t*)out, a.dout, lse, ndelta, nlse2, a.s, s);
  } else if (stage == Stage::kDkdv) {
    Buf in[5] = {{q, qb, "q"}, {k, kb, "k"}, {v, kb, "v"}, {dout, qb, "dout"}, {ws, need, "workspace"}};
    Buf outs[2] = {{dk, kb, "dk"}, {dv, kb, "dv"}};
    if ((st = check_buffers(in, 5, outs, 2))) return st;
    if ((st = injected_hip_error())) return st;
    e = s2a::launch_bwd_dkdv(a, nullptr, s);
  } else {
    Buf in[5] = {{q, qb, "q"}, {k, kb, "k"}, {v, kb, "v"}, {dout, qb, "dout"}, {ws, need, "workspace"}};
    Buf outs[1] = {{dq, qb, "dq"}};
    if ((st = check_buffers(in, 5, outs, 1))) return st;
    if ((st = injected_hip_error())) return st;
    e = s2a::launch_bwd_dq(a, nullptr, s);
  }
  if (e != hipSuccess) return hip_fail(e, "backward stage");
  return S2ATTN_OK;
}

size_t fwd_rope_ws(int B, int N, int H, int Hkv, int D) {
  if (B <= 0 || N <= 0 || Hkv <= 0 || D <= 0) return 0;
  (void)H;
  return round_up(q_bytes(B, N, Hkv, D));
}

size_t bwd_ws(int B, int N, int H, int Hkv, int D, bool rope) {
  if (B <= 0 || N <= 0 || H <= 0 || Hkv <= 0 || D <= 0) return 0;
  size_t n = 2 * round_up(stat_bytes(B, N, H));
  if (rope) n += round_up(q_bytes(B, N, H, D)) + round_up(q_bytes(B, N, Hkv, D));
  return n;
}

// Device scratch of the entry point that allocates nothing
// (s2attn_bwd_noalloc): the backward's two row statistics.  One copy per GPU
// the library runs on, held until the process ends.  In host code `scratch`
// is only a stand-in for the device symbol; its device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
constexpr size_t kScratchBytes = size_t(32) << 20;
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of this device's scratch, looked up on the first call on it.
int scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(S2ATTN_EUNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (ptr == nullptr || ((uintptr_t)ptr & (kAlign - 1)) != 0)
      return fail(S2ATTN_EHIP, "scratch address is null or not 256-byte aligned");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return S2ATTN_OK;
}

int do_bwd_noalloc(const void* q, const void* k, const void* v, const void* out, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv, int B, int N, int H, int Hkv, int D, int G, int shift,
                   void* stream) {
  int st = check_shape(B, N, H, Hkv, D, G, shift);
  if (st) return st;
  if (B == 0 || N == 0) return S2ATTN_OK;
  const size_t need = bwd_ws(B, N, H, Hkv, D, false);
  if (need > kScratchBytes)
    return fail(S2ATTN_EINVAL, "s2attn_bwd_noalloc: the row statistics need " + std::to_string(need) +
                                   " bytes, beyond its scratch of " + std::to_string(kScratchBytes) +
                                   " (B*H*N must stay at or below " + std::to_string(kScratchBytes / 8) + ")");
  if ((st = injected_hip_error())) return st;
  void* ws = nullptr;
  if ((st = scratch_for_current_device(&ws))) return st;
  return do_bwd(q, k, v, out, lse, dout, dq, dk, dv, B, N, H, Hkv, D, G, shift, nullptr, ws, kScratchBytes, stream);
}

}  // namespace

extern "C" {

int s2attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int N, int H, int Hkv,
               int D, int G, int shift, void* stream) {
  return guarded([&] { return do_fwd(q, k, v, out, lse, B, N, H, Hkv, D, G, shift, nullptr, nullptr, 0, stream); });
}

size_t s2attn_bwd_workspace_size(int B, int N, int H, int Hkv, int D) { return bwd_ws(B, N, H, Hkv, D, false); }

int s2attn_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse, const void* dout,
               void* dq, void* dk, void* dv, int B, int N, int H, int Hkv, int D, int G, int shift, void* workspace,
               size_t workspace_bytes, void* stream) {
  return guarded([&] {
    return do_bwd(q, k, v, out, lse, dout, dq, dk, dv, B, N, H, Hkv, D, G, shift, nullptr, workspace,
                  workspace_bytes, stream);
  });
}

int s2attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* out, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, int B, int N, int H, int Hkv, int D, int G,
                       int shift, void* stream) {
  return guarded([&] {
    return do_bwd_noalloc(q, k, v, out, lse, dout, dq, dk, dv, B, N, H, Hkv, D, G, shift, stream);
  });
}

int s2attn_bwd_preprocess(const void* out, const void* dout, const float* lse, int B, int N, int H, int D,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return guarded([&] {
    return do_bwd_stage(Stage::kPre, nullptr, nullptr, nullptr, out, lse, dout, nullptr, nullptr, nullptr, B, N, H,
                        H, D, 1, 0, workspace, workspace_bytes, stream);
  });
}

int s2attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, void* dk, void* dv, int B, int N,
                    int H, int Hkv, int D, int G, int shift, const void* workspace, size_t workspace_bytes,
                    void* stream) {
  return guarded([&] {
    return do_bwd_stage(Stage::kDkdv, q, k, v, nullptr, nullptr, dout, nullptr, dk, dv, B, N, H, Hkv, D, G, shift,
                        workspace, workspace_bytes, stream);
  });
}

int s2attn_bwd_dq(const void* q, const void* k, const void* v, const void* dout, void* dq, int B, int N, int H,
                  int Hkv, int D, int G, int shift, const void* workspace, size_t workspace_bytes, void* stream) {
  return guarded([&] {
    return do_bwd_stage(Stage::kDq, q, k, v, nullptr, nullptr, dout, dq, nullptr, nullptr, B, N, H, Hkv, D, G, shift,
                        workspace, workspace_bytes, stream);
  });
}

size_t s2attn_fwd_rope_workspace_size(int B, int N, int H, int Hkv, int D) { return fwd_rope_ws(B, N, H, Hkv, D); }

int s2attn_fwd_rope(const void* q, const void* k, const void* v, void* out, float* lse, int B, int N, int H,
                    int Hkv, int D, int G, int shift, double rope_base, double pos_scale, void* workspace,
                    size_t workspace_bytes, void* stream) {
  const double rope[2] = {rope_base, pos_scale};
  return guarded([&] {
    return do_fwd(q, k, v, out, lse, B, N, H, Hkv, D, G, shift, rope, workspace, workspace_bytes, stream);
  });
}

size_t s2attn_bwd_rope_workspace_size(int B, int N, int H, int Hkv, int D) { return bwd_ws(B, N, H, Hkv, D, true); }

int s2attn_bwd_rope(const void* q, const void* k, const void* v, const void* out, const float* lse,
                    const void* dout, void* dq, void* dk, void* dv, int B, int N, int H, int Hkv, int D, int G,
                    int shift, double rope_base, double pos_scale, void* workspace, size_t workspace_bytes,
                    void* stream) {
  const double rope[2] = {rope_base, pos_scale};
  return guarded([&] {
    return do_bwd(q, k, v, out, lse, dout, dq, dk, dv, B, N, H, Hkv, D, G, shift, rope, workspace,
                  workspace_bytes, stream);
  });
}

int s2attn_fwd_ex(const void* q, const void* k, const void* v, void* out, float* lse, int B, int N, int H,
                  int Hkv, int D, int G, int shift, int head_pattern, double rope_base, double pos_scale,
                  void* workspace, size_t workspace_bytes, void* stream) {
  const double rope[2] = {rope_base, pos_scale};
  return guarded([&] {
    return do_fwd(q, k, v, out, lse, B, N, H, Hkv, D, G, shift, rope_base != 0.0 ? rope : nullptr, workspace,
                  workspace_bytes, stream, head_pattern);
  });
}

int s2attn_bwd_ex(const void* q, const void* k, const void* v, const void* out, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, int B, int N, int H, int Hkv, int D, int G, int shift,
                  int head_pattern, double rope_base, double pos_scale, void* workspace, size_t workspace_bytes,
                  void* stream) {
  const double rope[2] = {rope_base, pos_scale};
  return guarded([&] {
    return do_bwd(q, k, v, out, lse, dout, dq, dk, dv, B, N, H, Hkv, D, G, shift,
                  rope_base != 0.0 ? rope : nullptr, workspace, workspace_bytes, stream, head_pattern);
  });
}

size_t s2attn_lora_qkv_workspace_size(int M, int r) {
  if (M <= 0 || r <= 0) return 0;
  return round_up((size_t)M * 3 * r * 2);
}

int s2attn_lora_qkv_fwd(const void* x, int M, int d_in, const void* wq_t, const void* wk_t, const void* wv_t,
                        int width_q, int width_kv, const void* aq_t, const void* ak_t, const void* av_t,
                        const void* bq_t, const void* bk_t, const void* bv_t, int r, double scale, void* q,
                        void* k, void* v, void* workspace, size_t workspace_bytes, void* stream) {
  return guarded([&] {
    if (M < 0) return fail(S2ATTN_EINVAL, "M must be >= 0");
    if (d_in < 64 || d_in % 64 != 0 || d_in > (1 << 20))
      return fail(S2ATTN_EINVAL, "d_in must be a multiple of 64 in [64, 2^20]");
    if (width_q < 64 || width_q % 64 != 0 || width_kv < 64 || width_kv % 64 != 0)
      return fail(S2ATTN_EINVAL, "width_q and width_kv must be multiples of 64 (>= 64)");
    if (r < 0 || r > 1024 || r % 8 != 0) return fail(S2ATTN_EINVAL, "r must be 0 or a multiple of 8 up to 1024");
    if (!std::isfinite(scale)) return fail(S2ATTN_EINVAL, "scale must be finite");
    const double tiles = std::ceil(M / 256.0) *
                         (double)(s2a::lora_col_tiles(width_q) + 2 * s2a::lora_col_tiles(width_kv));
    if (tiles > 2147483647.0) return fail(S2ATTN_EINVAL, "too many work items for one launch");
    if (M == 0) return (int)S2ATTN_OK;
    const size_t xb = (size_t)M * d_in * 2;
    const size_t wqb = (size_t)width_q * d_in * 2, wkb = (size_t)width_kv * d_in * 2;
    const size_t ab = (size_t)r * d_in * 2, bqb = (size_t)width_q * r * 2, bkb = (size_t)width_kv * r * 2;
    const size_t yqb = (size_t)M * width_q * 2, ykb = (size_t)M * width_kv * 2;
    const size_t need = s2attn_lora_qkv_workspace_size(M, r);
    if (r > 0) {
      if (workspace == nullptr) return fail(S2ATTN_EINVAL, "workspace is NULL");
      if (workspace_bytes < need)
        return fail(S2ATTN_EINVAL, "workspace too small: need " + std::to_string(need) + " bytes");
      if (((uintptr_t)workspace & (kAlign - 1)) != 0) return fail(S2ATTN_EINVAL, "workspace is not 256-byte aligned");
      const Buf in[] = {{x, xb, "x"},     {wq_t, wqb, "wq_t"}, {wk_t, wkb, "wk_t"}, {wv_t, wkb, "wv_t"},
                        {aq_t, ab, "aq_t"}, {ak_t, ab, "ak_t"},  {av_t, ab, "av_t"},  {bq_t, bqb, "bq_t"},
                        {bk_t, bkb, "bk_t"}, {bv_t, bkb, "bv_t"}};
      const Buf out[] = {{q, yqb, "q"}, {k, ykb, "k"}, {v, ykb, "v"}, {workspace, need, "workspace"}};
      int st = check_buffers(in, 10, out, 4);
      if (st) return st;
    } else {
      const Buf in[] = {{x, xb, "x"}, {wq_t, wqb, "wq_t"}, {wk_t, wkb, "wk_t"}, {wv_t, wkb, "wv_t"}};
      const Buf out[] = {{q, yqb, "q"}, {k, ykb, "k"}, {v, ykb, "v"}};
      int st = check_buffers(in, 4, out, 3);
      if (st) return st;
    }
    s2a::LoraQkvArgs a{};
    a.x = (const uint16_t*)x;
    a.M = M;
    a.K = d_in;
    const void* wt[3] = {wq_t, wk_t, wv_t};
    const void* at[3] = {aq_t, ak_t, av_t};
    const void* bt[3] = {bq_t, bk_t, bv_t};
    void* y[3] = {q, k, v};
    for (int p = 0; p < 3; ++p) {
      a.wt[p] = (const uint16_t*)wt[p];
      a.at[p] = r > 0 ? (const uint16_t*)at[p] : nullptr;
      a.bt[p] = r > 0 ? (const uint16_t*)bt[p] : nullptr;
      a.width[p] = p == 0 ? width_q : width_kv;
      a.y[p] = (uint16_t*)y[p];
    }
    a.r = r;
    a.scale = (float)scale;
    a.t = r > 0 ? (uint16_t*)workspace : nullptr;
    if (int ist = injected_hip_error()) return ist;
    hipError_t e = s2a::launch_lora_qkv(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "lora_qkv launch");
    return (int)S2ATTN_OK;
  });
}

size_t s2attn_lora_qkv_bwd_workspace_size(int M, int d_in, int width_q, int width_kv, int r) {
  if (M <= 0 || r <= 0) return 0;
  const size_t imax = (size_t)std::max(d_in, std::max(width_q, width_kv));
  return round_up((size_t)M * 3 * r * 2) + round_up((size_t)s2a::lora_bwd_splits(M) * imax * r * 4);
}

int s2attn_lora_qkv_bwd(const void* x, int M, int d_in, const void* wq_t, const void* wk_t, const void* wv_t,
                        int width_q, int width_kv, const void* aq_t, const void* ak_t, const void* av_t,
                        const void* bq_t, const void* bk_t, const void* bv_t, int r, double scale, const void* t,
                        const void* dq, const void* dk, const void* dv, void* dx, void* daq_t, void* dak_t,
                        void* dav_t, void* dbq_t, void* dbk_t, void* dbv_t, void* workspace, size_t workspace_bytes,
                        void* stream) {
  return guarded([&] {
    if (M < 0) return fail(S2ATTN_EINVAL, "M must be >= 0");
    if (d_in < 64 || d_in % 64 != 0 || d_in > (1 << 20))
      return fail(S2ATTN_EINVAL, "d_in must be a multiple of 64 in [64, 2^20]");
    if (width_q < 64 || width_q % 64 != 0 || width_kv < 64 || width_kv % 64 != 0 || width_q > (1 << 20) ||
        width_kv > (1 << 20))
      return fail(S2ATTN_EINVAL, "width_q and width_kv must be multiples of 64 in [64, 2^20]");
    if (r < 0 || r > 1024 || r % 8 != 0) return fail(S2ATTN_EINVAL, "r must be 0 or a multiple of 8 up to 1024");
    if (!std::isfinite(scale)) return fail(S2ATTN_EINVAL, "scale must be finite");
    if (std::ceil(M / 256.0) * std::ceil(std::max(d_in, std::max(width_q, width_kv)) / 256.0) > 2147483647.0 ||
        (double)s2a::lora_bwd_splits(M) * std::ceil(std::max(d_in, std::max(width_q, width_kv)) / 128.0) * std::ceil(r / 64.0) >
            2147483647.0)
      return fail(S2ATTN_EINVAL, "too many work items for one launch");
    if (M == 0) return (int)S2ATTN_OK;
    const size_t xb = (size_t)M * d_in * 2;
    const size_t wqb = (size_t)width_q * d_in * 2, wkb = (size_t)width_kv * d_in * 2;
    const size_t ab = (size_t)r * d_in * 2, bqb = (size_t)width_q * r * 2, bkb = (size_t)width_kv * r * 2;
    const size_t yqb = (size_t)M * width_q * 2, ykb = (size_t)M * width_kv * 2;
    const size_t tb = (size_t)M * 3 * r * 2;
    const size_t need = s2attn_lora_qkv_bwd_workspace_size(M, d_in, width_q, width_kv, r);
    if (r > 0) {
      if (workspace == nullptr) return fail(S2ATTN_EINVAL, "workspace is NULL");
      if (workspace_bytes < need)
        return fail(S2ATTN_EINVAL, "workspace too small: need " + std::to_string(need) + " bytes");
      if (((uintptr_t)workspace & (kAlign - 1)) != 0) return fail(S2ATTN_EINVAL, "workspace is not 256-byte aligned");
      const Buf in[] = {{x, xb, "x"},       {wq_t, wqb, "wq_t"}, {wk_t, wkb, "wk_t"}, {wv_t, wkb, "wv_t"},
                        {aq_t, ab, "aq_t"}, {ak_t, ab, "ak_t"},  {av_t, ab, "av_t"},  {bq_t, bqb, "bq_t"},
                        {bk_t, bkb, "bk_t"}, {bv_t, bkb, "bv_t"}, {t, tb, "t"},        {dq, yqb, "dq"},
                        {dk, ykb, "dk"},    {dv, ykb, "dv"}};
      const Buf out[] = {{dx, xb, "dx"},      {daq_t, ab, "daq_t"}, {dak_t, ab, "dak_t"},
                         {dav_t, ab, "dav_t"}, {dbq_t, bqb, "dbq_t"}, {dbk_t, bkb, "dbk_t"},
                         {dbv_t, bkb, "dbv_t"}, {workspace, need, "workspace"}};
      int st = check_buffers(in, 14, out, 8);
      if (st) return st;
    } else {
      const Buf in[] = {{x, xb, "x"},    {wq_t, wqb, "wq_t"}, {wk_t, wkb, "wk_t"}, {wv_t, wkb, "wv_t"},
                        {dq, yqb, "dq"}, {dk, ykb, "dk"},     {dv, ykb, "dv"}};
      const Buf out[] = {{dx, xb, "dx"}};
      int st = check_buffers(in, 7, out, 1);
      if (st) return st;
    }
    s2a::LoraQkvBwdArgs a{};
    a.x = (const uint16_t*)x;
    a.M = M;
    a.K = d_in;
    const void* wt[3] = {wq_t, wk_t, wv_t};
    const void* at[3] = {aq_t, ak_t, av_t};
    const void* bt[3] = {bq_t, bk_t, bv_t};
    const void* dy[3] = {dq, dk, dv};
    void* dat[3] = {daq_t, dak_t, dav_t};
    void* dbt[3] = {dbq_t, dbk_t, dbv_t};
    for (int p = 0; p < 3; ++p) {
      a.wt[p] = (const uint16_t*)wt[p];
      a.at[p] = r > 0 ? (const uint16_t*)at[p] : nullptr;
      a.bt[p] = r > 0 ? (const uint16_t*)bt[p] : nullptr;
      a.width[p] = p == 0 ? width_q : width_kv;
      a.dy[p] = (const uint16_t*)dy[p];
      a.dat[p] = r > 0 ? (uint16_t*)dat[p] : nullptr;
      a.dbt[p] = r > 0 ? (uint16_t*)dbt[p] : nullptr;
    }
    a.r = r;
    a.scale = (float)scale;
    a.t = r > 0 ? (const uint16_t*)t : nullptr;
    a.dx = (uint16_t*)dx;
    if (r > 0) {
      a.dts = (uint16_t*)workspace;
      a.part = (float*)((char*)workspace + round_up(tb));
    }
    if (int ist = injected_hip_error()) return ist;
    hipError_t e = s2a::launch_lora_qkv_bwd(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "lora_qkv_bwd launch");
    return (int)S2ATTN_OK;
  });
}

const char* s2attn_strerror(int status) {
  switch (status) {
    case S2ATTN_OK: return "success";
    case S2ATTN_EINVAL: return "invalid argument";
    case S2ATTN_EUNSUPPORTED: return "unsupported configuration";
    case S2ATTN_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* s2attn_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
