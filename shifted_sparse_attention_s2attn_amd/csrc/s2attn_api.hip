// C ABI of libs2attn: host-side validation, workspace sizing and launch.
// Every check runs on the host before any HIP call, so a rejected call
// launches nothing.  The library keeps no state, apart from the per-device
// address of the scratch array of s2attn_bwd_noalloc (at the end of this file).
#include "s2attn.h"

#include <math.h>
#include <atomic>
#include <initializer_list>
#include <mutex>
#include <stdint.h>
#include "s2attn_common.h"

namespace s2a {
template <typename T, int D>
hipError_t launch_rope(const void*, void*, int, int, int, double, double, int, hipStream_t);
template <typename T, int D>
hipError_t launch_fwd(const void*, const void*, const void*, void*, float*, int, int, int, int, int, int, int,
                      hipStream_t);
template <typename T, int D>
hipError_t launch_bwd_prep(const void*, const void*, const float*, float*, float*, int, int, int, hipStream_t);
template <typename T, int D>
hipError_t launch_bwd_dkdv(const void*, const void*, const void*, const void*, const float*, const float*, void*,
                           void*, int, int, int, int, int, int, int, hipStream_t, float*);
template <typename T, int D>
hipError_t launch_bwd_dq(const void*, const void*, const void*, const void*, const float*, const float*, void*,
                         int, int, int, int, int, int, int, hipStream_t);
template <typename T, int D>
hipError_t launch_bwd_prep_dq(const void*, const void*, const void*, const void*, const float*, const void*,
                              float*, float*, void*, int, int, int, int, int, int, int, hipStream_t);
template <int D>
hipError_t launch_fwd_rope(const void*, const void*, const void*, void*, float*, void*, int, int, int, int, int, int,
                           int, double, double, hipStream_t);
template <int D>
hipError_t launch_bwd_rope(const void*, const void*, const void*, const void*, const float*, const void*, float*,
                           float*, void*, void*, void*, int, int, int, int, int, int, int, double, double,
                           hipStream_t, float*);
}  // namespace s2a

namespace {

constexpr int kTileRows = 128;   // query rows per forward workgroup = key rows per backward workgroup

// Whole groups of whole 128-row tiles.  Other shapes (G not dividing N, so the
// last group is short, or G not a multiple of 128) take the kernels' EDGE
// instantiations, which address tiles row by row where they cross a group end,
// the wrap point or the sequence end.
bool aligned(int N, int G) { return N % G == 0 && G % kTileRows == 0; }

// Sizes only (no pointers).  B == 0 or N == 0 is a valid, empty problem.
int check_problem(int B, int H, int Hkv, int N, int d, int G, int shift_heads, int dtype) {
  if (B < 0 || N < 0 || H <= 0 || Hkv <= 0 || d <= 0 || G <= 0) return S2ATTN_ERR_SHAPE;
  if (N > 0 && G > N) return S2ATTN_ERR_SHAPE;
  if (shift_heads < 0 || shift_heads > H) return S2ATTN_ERR_SHAPE;
  if (H % Hkv != 0) return S2ATTN_ERR_SHAPE;
  // one-dimensional grids of (batch, head, group, 128-row tile) blocks
  const size_t blocks = (size_t)B * H * (size_t)((N + G - 1) / G) * (size_t)((G + kTileRows - 1) / kTileRows);
  if (blocks > (size_t)INT32_MAX) return S2ATTN_ERR_UNSUPPORTED;
  // the bf16 kernels address a 64-row tile with 32-bit byte offsets from its
  // first row: 64 rows of q (H * d elements each, the widest tensor) < 2^31 bytes
  if ((size_t)H * (size_t)d >= ((size_t)1 << 24)) return S2ATTN_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return S2ATTN_ERR_UNSUPPORTED;
  if (dtype != S2ATTN_BF16 && dtype != S2ATTN_F32) return S2ATTN_ERR_UNSUPPORTED;
  return S2ATTN_OK;
}

// A key/value head read by both shifted and unshifted query heads: one dK/dV
// launch tiles its keys in the first head's frame, and the other frame, G/2
// away, must then cut them into whole tiles of whole groups.  Otherwise dK/dV
// runs in two passes (unshifted heads, then shifted ones), the first leaving
// its fp32 sums in the workspace for the second.
bool two_pass_dkdv(int H, int Hkv, int N, int G, int shift_heads) {
  const int r = H / Hkv;
  return r > 1 && (H - shift_heads) % r != 0 && (!aligned(N, G) || (G / 2) % kTileRows != 0);
}

bool empty_problem(int B, int N) { return B == 0 || N == 0; }

// Element tensors are read and written in 16-byte vectors; lse takes 4-byte
// scalars.  Checked after the NULL checks, before any HIP call.
bool misaligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (reinterpret_cast<uintptr_t>(p) & 15) return true;
  return false;
}
bool misaligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) != 0; }

// The wrap options: the main method's roll, the split option (the wrap group
// cut where the roll wraps) and the swap option (the wrap group's front tokens
// first), on every shape.
int check_wrap(int wrap, int N, int G) {
  (void)N;
  (void)G;
  return (wrap == S2ATTN_WRAP_ROLL || wrap == S2ATTN_WRAP_SPLIT || wrap == S2ATTN_WRAP_SWAP) ? S2ATTN_OK
                                                                                              : S2ATTN_ERR_UNSUPPORTED;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Rotary embedding parameters: a finite, non-negative position scale and a
// finite base above 1.
bool bad_rope(double pos_scale, double base) {
  return !isfinite(pos_scale) || pos_scale < 0 || !isfinite(base) || !(base > 1);
}

}  // namespace

extern "C" {

int s2attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int Hkv, int N, int d, int G, int shift_heads, int wrap, int dtype, void* stream) {
  int st = check_problem(B, H, Hkv, N, d, G, shift_heads, dtype);
  if (st == S2ATTN_OK) st = check_wrap(wrap, N, G);
  if (st != S2ATTN_OK) return st;
  if (empty_problem(B, N)) return S2ATTN_OK;
  if (!q || !k || !v || !o || !lse) return S2ATTN_ERR_NULL;
  if (misaligned16({q, k, v, o}) || misaligned4(lse)) return S2ATTN_ERR_ALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == S2ATTN_BF16) {
    e = d == 64 ? s2a::launch_fwd<s2a::bf16, 64>(q, k, v, o, lse, B, H, Hkv, N, G, shift_heads, wrap, s)
                : s2a::launch_fwd<s2a::bf16, 128>(q, k, v, o, lse, B, H, Hkv, N, G, shift_heads, wrap, s);
  } else {
    e = d == 64 ? s2a::launch_fwd<float, 64>(q, k, v, o, lse, B, H, Hkv, N, G, shift_heads, wrap, s)
                : s2a::launch_fwd<float, 128>(q, k, v, o, lse, B, H, Hkv, N, G, shift_heads, wrap, s);
  }
  return e == hipSuccess ? S2ATTN_OK : S2ATTN_ERR_HIP;
}

int s2attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int Hkv, int N, int d, int G, int shift_heads, int dtype, void* stream) {
  return s2attn_fwd_ex(q, k, v, o, lse, B, H, Hkv, N, d, G, shift_heads, S2ATTN_WRAP_ROLL, dtype, stream);
}

size_t s2attn_bwd_workspace_bytes(int B, int H, int Hkv, int N, int d, int G, int shift_heads, int dtype) {
  if (check_problem(B, H, Hkv, N, d, G, shift_heads, dtype) != S2ATTN_OK) return 0;
  const size_t rows = 2 * align256((size_t)B * H * N * sizeof(float));
  if (!two_pass_dkdv(H, Hkv, N, G, shift_heads)) return rows;
  return rows + align256(2 * (size_t)B * N * Hkv * d * sizeof(float));
}

}  // extern "C"

namespace {

// Workspace: -Dvec [B,H,N] | lse*log2(e) [B,H,N] | (two-pass dK/dV only) the first
// pass's dK, dV sums [2][B,N,Hkv,d], fp32.
struct Workspace {
  float* dvec;
  float* lse2;
  float* part;   // NULL: one dK/dV pass
};

int check_workspace(void* workspace, size_t workspace_bytes, int B, int H, int Hkv, int N, int d, int G,
                    int shift_heads, int dtype, Workspace* ws) {
  const size_t need = s2attn_bwd_workspace_bytes(B, H, Hkv, N, d, G, shift_heads, dtype);
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return S2ATTN_ERR_WORKSPACE;
  ws->dvec = static_cast<float*>(workspace);
  ws->lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + align256((size_t)B * H * N * sizeof(float)));
  ws->part = two_pass_dkdv(H, Hkv, N, G, shift_heads)
                 ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                            2 * align256((size_t)B * H * N * sizeof(float)))
                 : nullptr;
  return S2ATTN_OK;
}

// Dispatch a launcher template over (dtype, d).
template <template <typename, int> class L, typename... A>
hipError_t dispatch(int dtype, int d, A... a) {
  if (dtype == S2ATTN_BF16) return d == 64 ? L<s2a::bf16, 64>::run(a...) : L<s2a::bf16, 128>::run(a...);
  return d == 64 ? L<float, 64>::run(a...) : L<float, 128>::run(a...);
}

template <typename T, int D>
struct Prep {
  static hipError_t run(const void* o, const void* dO, const float* lse, Workspace ws, int B, int H, int N,
                        hipStream_t s) {
    return s2a::launch_bwd_prep<T, D>(o, dO, lse, ws.dvec, ws.lse2, B, H, N, s);
  }
};
template <typename T, int D>
struct Dkdv {
  static hipError_t run(const void* q, const void* k, const void* v, const void* dO, void* dk, void* dv,
                        Workspace ws, int B, int H, int Hkv, int N, int G, int S, int wrap, hipStream_t s) {
    return s2a::launch_bwd_dkdv<T, D>(q, k, v, dO, ws.lse2, ws.dvec, dk, dv, B, H, Hkv, N, G, S, wrap, s, ws.part);
  }
};
template <typename T, int D>
struct Dq {
  static hipError_t run(const void* q, const void* k, const void* v, const void* dO, void* dq, Workspace ws,
                        int B, int H, int Hkv, int N, int G, int S, int wrap, hipStream_t s) {
    return s2a::launch_bwd_dq<T, D>(q, k, v, dO, ws.lse2, ws.dvec, dq, B, H, Hkv, N, G, S, wrap, s);
  }
};

template <typename T, int D>
struct PrepDq {
  static hipError_t run(const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const void* dO, void* dq, Workspace ws, int B, int H, int Hkv, int N, int G, int S, int wrap,
                        hipStream_t s) {
    return s2a::launch_bwd_prep_dq<T, D>(q, k, v, o, lse, dO, ws.lse2, ws.dvec, dq, B, H, Hkv, N, G, S, wrap, s);
  }
};

int status_of(hipError_t e) { return e == hipSuccess ? S2ATTN_OK : S2ATTN_ERR_HIP; }

}  // namespace

extern "C" {

int s2attn_bwd_prep(const void* o, const float* lse, const void* dO, void* workspace, size_t workspace_bytes,
                    int B, int H, int Hkv, int N, int d, int G, int shift_heads, int dtype, void* stream) {
  int st = check_problem(B, H, Hkv, N, d, G, shift_heads, dtype);
  if (st != S2ATTN_OK) return st;
  if (empty_problem(B, N)) return S2ATTN_OK;
  if (!o || !lse || !dO) return S2ATTN_ERR_NULL;
  if (misaligned16({o, dO}) || misaligned4(lse)) return S2ATTN_ERR_ALIGN;
  Workspace ws;
  st = check_workspace(workspace, workspace_bytes, B, H, Hkv, N, d, G, shift_heads, dtype, &ws);
  if (st != S2ATTN_OK) return st;
  return status_of(dispatch<Prep>(dtype, d, o, dO, lse, ws, B, H, N, reinterpret_cast<hipStream_t>(stream)));
}

int s2attn_bwd_dkdv_ex(const void* q, const void* k, const void* v, const void* dO, void* dk, void* dv,
                       void* workspace, size_t workspace_bytes,
                       int B, int H, int Hkv, int N, int d, int G, int shift_heads, int wrap, int dtype,
                       void* stream) {
  int st = check_problem(B, H, Hkv, N, d, G, shift_heads, dtype);
  if (st == S2ATTN_OK) st = check_wrap(wrap, N, G);
  if (st != S2ATTN_OK) return st;
  if (empty_problem(B, N)) return S2ATTN_OK;
  if (!q || !k || !v || !dO || !dk || !dv) return S2ATTN_ERR_NULL;
  if (misaligned16({q, k, v, dO, dk, dv})) return S2ATTN_ERR_ALIGN;
  Workspace ws;
  st = check_workspace(workspace, workspace_bytes, B, H, Hkv, N, d, G, shift_heads, dtype, &ws);
  if (st != S2ATTN_OK) return st;
  return status_of(dispatch<Dkdv>(dtype, d, q, k, v, dO, dk, dv, ws, B, H, Hkv, N, G, shift_heads, wrap,
                                  reinterpret_cast<hipStream_t>(stream)));
}

int s2attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO, void* dk, void* dv,
                    void* workspace, size_t workspace_bytes,
                    int B, int H, int Hkv, int N, int d, int G, int shift_heads, int dtype, void* stream) {
  return s2attn_bwd_dkdv_ex(q, k, v, dO, dk, dv, workspace, workspace_bytes, B, H, Hkv, N, d, G, shift_heads,
                            S2ATTN_WRAP_ROLL, dtype, stream);
}

int s2attn_bwd_dq_ex(const void* q, const void* k, const void* v, const void* dO, void* dq,
                     void* workspace, size_t workspace_bytes,
                     int B, int H, int Hkv, int N, int d, int G, int shift_heads, int wrap, int dtype,
                     void* stream) {
  int st = check_problem(B, H, Hkv, N, d, G, shift_heads, dtype);
  if (st == S2ATTN_OK) st = check_wrap(wrap, N, G);
  if (st != S2ATTN_OK) return st;
  if (empty_problem(B, N)) return S2ATTN_OK;
  if (!q || !k || !v || !dO || !dq) return S2ATTN_ERR_NULL;
  if (misaligned16({q, k, v, dO, dq})) return S2ATTN_ERR_ALIGN;
  Workspace ws;
  st = check_workspace(workspace, workspace_bytes, B, H, Hkv, N, d, G, shift_heads, dtype, &ws);
  if (st != S2ATTN_OK) return st;
  return status_of(dispatch<Dq>(dtype, d, q, k, v, dO, dq, ws, B, H, Hkv, N, G, shift_heads, wrap,
                                reinterpret_cast<hipStream_t>(stream)));
}

int s2attn_bwd_dq(const void* q, const void* k, const void* v, const void* dO, void* dq,
                  void* workspace, size_t workspace_bytes,
                  int B, int H, int Hkv, int N, int d, int G, int shift_heads, int dtype, void* stream) {
  return s2attn_bwd_dq_ex(q, k, v, dO, dq, workspace, workspace_bytes, B, H, Hkv, N, d, G, shift_heads,
                          S2ATTN_WRAP_ROLL, dtype, stream);
}

int s2attn_bwd_prep_dq(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dO, void* dq, void* workspace, size_t workspace_bytes,
                       int B, int H, int Hkv, int N, int d, int G, int shift_heads, int wrap, int dtype,
                       void* stream) {
  int st = check_problem(B, H, Hkv, N, d, G, shift_heads, dtype);
  if (st == S2ATTN_OK) st = check_wrap(wrap, N, G);
  if (st != S2ATTN_OK) return st;
  if (empty_problem(B, N)) return S2ATTN_OK;
  if (!q || !k || !v || !o || !lse || !dO || !dq) return S2ATTN_ERR_NULL;
  if (misaligned16({q, k, v, o, dO, dq}) || misaligned4(lse)) return S2ATTN_ERR_ALIGN;
  Workspace ws;
  st = check_workspace(workspace, workspace_bytes, B, H, Hkv, N, d, G, shift_heads, dtype, &ws);
  if (st != S2ATTN_OK) return st;
  return status_of(dispatch<PrepDq>(dtype, d, q, k, v, o, lse, dO, dq, ws, B, H, Hkv, N, G, shift_heads, wrap,
                                    reinterpret_cast<hipStream_t>(stream)));
}

int s2attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                  void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                  int B, int H, int Hkv, int N, int d, int G, int shift_heads, int wrap, int dtype, void* stream) {
  int st = check_problem(B, H, Hkv, N, d, G, shift_heads, dtype);
  if (st == S2ATTN_OK) st = check_wrap(wrap, N, G);
  if (st != S2ATTN_OK) return st;
  if (empty_problem(B, N)) return S2ATTN_OK;
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return S2ATTN_ERR_NULL;
  if (misaligned16({q, k, v, o, dO, dq, dk, dv}) || misaligned4(lse)) return S2ATTN_ERR_ALIGN;
  Workspace ws;
  st = check_workspace(workspace, workspace_bytes, B, H, Hkv, N, d, G, shift_heads, dtype, &ws);
  if (st != S2ATTN_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // prep fused into dq (it writes the workspace), then dK/dV
  hipError_t e = dispatch<PrepDq>(dtype, d, q, k, v, o, lse, dO, dq, ws, B, H, Hkv, N, G, shift_heads, wrap, s);
  if (e == hipSuccess)
    e = dispatch<Dkdv>(dtype, d, q, k, v, dO, dk, dv, ws, B, H, Hkv, N, G, shift_heads, wrap, s);
  return status_of(e);
}

int s2attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
               void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
               int B, int H, int Hkv, int N, int d, int G, int shift_heads, int dtype, void* stream) {
  return s2attn_bwd_ex(q, k, v, o, lse, dO, dq, dk, dv, workspace, workspace_bytes, B, H, Hkv, N, d, G,
                       shift_heads, S2ATTN_WRAP_ROLL, dtype, stream);
}

int s2attn_fwd_rope(const void* q, const void* k_rot, const void* v, void* o, float* lse, void* q_rot,
                    int B, int H, int Hkv, int N, int d, int G, int shift_heads, int wrap,
                    double pos_scale, double base, int dtype, void* stream) {
  int st = check_problem(B, H, Hkv, N, d, G, shift_heads, dtype);
  if (st == S2ATTN_OK) st = check_wrap(wrap, N, G);
  if (st != S2ATTN_OK) return st;
  if (dtype != S2ATTN_BF16 || bad_rope(pos_scale, base)) return S2ATTN_ERR_UNSUPPORTED;
  if (empty_problem(B, N)) return S2ATTN_OK;
  if (!q || !k_rot || !v || !o || !lse || !q_rot) return S2ATTN_ERR_NULL;
  if (misaligned16({q, k_rot, v, o, q_rot}) || misaligned4(lse)) return S2ATTN_ERR_ALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e =
      d == 64 ? s2a::launch_fwd_rope<64>(q, k_rot, v, o, lse, q_rot, B, H, Hkv, N, G, shift_heads, wrap, pos_scale,
                                         log2(base), s)
              : s2a::launch_fwd_rope<128>(q, k_rot, v, o, lse, q_rot, B, H, Hkv, N, G, shift_heads, wrap, pos_scale,
                                          log2(base), s);
  return status_of(e);
}

int s2attn_bwd_rope(const void* q_rot, const void* k_rot, const void* v, const void* o, const float* lse,
                    const void* dO, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                    int B, int H, int Hkv, int N, int d, int G, int shift_heads, int wrap,
                    double pos_scale, double base, int dtype, void* stream) {
  int st = check_problem(B, H, Hkv, N, d, G, shift_heads, dtype);
  if (st == S2ATTN_OK) st = check_wrap(wrap, N, G);
  if (st != S2ATTN_OK) return st;
  if (dtype != S2ATTN_BF16 || bad_rope(pos_scale, base)) return S2ATTN_ERR_UNSUPPORTED;
  if (empty_problem(B, N)) return S2ATTN_OK;
  if (!q_rot || !k_rot || !v || !o || !lse || !dO || !dq || !dk || !dv) return S2ATTN_ERR_NULL;
  if (misaligned16({q_rot, k_rot, v, o, dO, dq, dk, dv}) || misaligned4(lse)) return S2ATTN_ERR_ALIGN;
  Workspace ws;
  st = check_workspace(workspace, workspace_bytes, B, H, Hkv, N, d, G, shift_heads, dtype, &ws);
  if (st != S2ATTN_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e =
      d == 64 ? s2a::launch_bwd_rope<64>(q_rot, k_rot, v, o, lse, dO, ws.lse2, ws.dvec, dq, dk, dv, B, H, Hkv, N, G,
                                         shift_heads, wrap, pos_scale, log2(base), s, ws.part)
              : s2a::launch_bwd_rope<128>(q_rot, k_rot, v, o, lse, dO, ws.lse2, ws.dvec, dq, dk, dv, B, H, Hkv, N, G,
                                          shift_heads, wrap, pos_scale, log2(base), s, ws.part);
  return status_of(e);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// s2attn_bwd_noalloc: the backward's scratch in a file-scope device array.
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up per device with hipGetSymbolAddress and only
// that address is passed to kernels.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = 2 * (size_t)S2ATTN_NOALLOC_MAX_ROWS * sizeof(float);   // -Dvec | lse*log2(e)
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag scratch_once[kMaxDevices];
std::atomic<void*> scratch_ptr[kMaxDevices];

// Device address of this device's scratch array (the current device), looked
// up once per device; NULL if the lookup failed.
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(scratch_once[dev], [dev] {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) scratch_ptr[dev].store(p);
  });
  return scratch_ptr[dev].load();
}

}  // namespace

extern "C" {

int s2attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                       void* dq, void* dk, void* dv,
                       int B, int H, int Hkv, int N, int d, int G, int shift_heads, int wrap, int dtype,
                       void* stream) {
  int st = check_problem(B, H, Hkv, N, d, G, shift_heads, dtype);
  if (st == S2ATTN_OK) st = check_wrap(wrap, N, G);
  if (st != S2ATTN_OK) return st;
  const size_t rows = (size_t)B * H * N;
  if (rows > (size_t)S2ATTN_NOALLOC_MAX_ROWS) return S2ATTN_ERR_SCRATCH;
  // the workspace layout of s2attn_bwd_ex, inside the scratch array (a two-pass
  // dK/dV's partial sums included, where they fit)
  const size_t need = s2attn_bwd_workspace_bytes(B, H, Hkv, N, d, G, shift_heads, dtype);
  if (need > kScratchBytes) return S2ATTN_ERR_SCRATCH;
  if (empty_problem(B, N)) return S2ATTN_OK;
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return S2ATTN_ERR_NULL;
  if (misaligned16({q, k, v, o, dO, dq, dk, dv}) || misaligned4(lse)) return S2ATTN_ERR_ALIGN;
  void* base = scratch_address();
  if (!base) return S2ATTN_ERR_HIP;
  Workspace ws;
  st = check_workspace(base, need, B, H, Hkv, N, d, G, shift_heads, dtype, &ws);
  if (st != S2ATTN_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = dispatch<PrepDq>(dtype, d, q, k, v, o, lse, dO, dq, ws, B, H, Hkv, N, G, shift_heads, wrap, s);
  if (e == hipSuccess)
    e = dispatch<Dkdv>(dtype, d, q, k, v, dO, dk, dv, ws, B, H, Hkv, N, G, shift_heads, wrap, s);
  return status_of(e);
}

int s2attn_rope(const void* x, void* y, int B, int N, int Hx, int d, double pos_scale, double base,
                int inverse, int dtype, void* stream) {
  if (B < 0 || N < 0 || Hx <= 0 || d <= 0) return S2ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return S2ATTN_ERR_UNSUPPORTED;
  if (dtype != S2ATTN_BF16 && dtype != S2ATTN_F32) return S2ATTN_ERR_UNSUPPORTED;
  if (bad_rope(pos_scale, base) || (inverse != 0 && inverse != 1)) return S2ATTN_ERR_UNSUPPORTED;
  if (empty_problem(B, N)) return S2ATTN_OK;
  if (!x || !y) return S2ATTN_ERR_NULL;
  if (misaligned16({x, y})) return S2ATTN_ERR_ALIGN;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == S2ATTN_BF16)
    e = d == 64 ? s2a::launch_rope<s2a::bf16, 64>(x, y, B, N, Hx, pos_scale, base, inverse, s)
                : s2a::launch_rope<s2a::bf16, 128>(x, y, B, N, Hx, pos_scale, base, inverse, s);
  else
    e = d == 64 ? s2a::launch_rope<float, 64>(x, y, B, N, Hx, pos_scale, base, inverse, s)
                : s2a::launch_rope<float, 128>(x, y, B, N, Hx, pos_scale, base, inverse, s);
  return e == hipSuccess ? S2ATTN_OK : S2ATTN_ERR_HIP;
}

const char* s2attn_status_str(int status) {  switch (status) {
    case S2ATTN_OK: return "ok";
    case S2ATTN_ERR_NULL: return "a required pointer is NULL";
    case S2ATTN_ERR_SHAPE: return "invalid shape (a size < 0, H, Hkv, d or G <= 0, G > N, shift_heads outside [0,H], or H % Hkv != 0)";
    case S2ATTN_ERR_UNSUPPORTED: return "unsupported problem (d not 64/128, unknown dtype or wrap option, grid too large, H * d >= 2^24, a rotary scale, base or direction out of range, or an fp32 problem for the fused rotary calls)";
    case S2ATTN_ERR_HIP: return "HIP kernel launch failed";
    case S2ATTN_ERR_WORKSPACE: return "workspace missing, misaligned or smaller than s2attn_bwd_workspace_bytes()";
    case S2ATTN_ERR_ALIGN: return "a tensor pointer is misaligned (element tensors need 16 bytes, lse 4)";
    case S2ATTN_ERR_SCRATCH: return "the problem does not fit the library's scratch array (B * H * N above S2ATTN_NOALLOC_MAX_ROWS, or a two-pass dK/dV whose workspace exceeds the array)";
    default: return "unknown status";
  }
}

}  // extern "C"
