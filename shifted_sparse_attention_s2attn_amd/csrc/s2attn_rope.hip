// Rotary position embedding with Position Interpolation on q or k (gfx950).
//
// The step before the attention on the pages' fine-tuning path (page
// "LongLoRA: Efficient Fine-tuning of Long-Context Large Language Models",
// section 3.2 Phase 1 item 2, and "Training Procedure, Hyperparameters, and
// Dataset Configuration", "Model setup"): the pre-trained model's rotary
// position embeddings are rescaled by Position Interpolation, every position
// multiplied by original context / target context.  The rotation itself is
// the published rotary embedding in the rotate-half pairing: dimension i is
// paired with i + d/2 and turned by t = n * pos_scale * base^(-2i/d) at token n.
//
// An elementwise pass bound by HBM bandwidth (one read and one write of the
// tensor).  With the fused attention calls (s2attn_fwd_rope / s2attn_bwd_rope)
// only k takes this pass: q is turned in the forward kernel's registers, and dq
// and dk are turned back in the backward kernels' epilogues, with the helpers
// of s2attn_common.h, so both routes give the same rotated values.
//
// One thread owns 8 consecutive pairs (dimensions 8c .. 8c+7 and their
// partners d/2 + 8c ..) and strides over rows, so its 8 frequencies are
// computed once, in float64.  Angles are formed in float64, in revolutions,
// and reduced to [-1/2, 1/2] before the float32 sine and cosine: at positions
// near 10^5 a float32 angle would be off by ~10^-2 radians.  bf16 outputs take
// the hardware sine and cosine of revolutions (error far below the output's
// rounding); fp32 outputs take sincosf.
#include "s2attn_common.h"

namespace s2a {

// I: the row index type (32-bit while the row count allows it: cheaper division)
template <typename T, int D, typename I>
__global__ __launch_bounds__(256) void s2attn_rope_kernel(const T* x, T* y, I rows, int N, int Hx,
                                                          double pos_scale, double log2_base, int inverse) {
  constexpr int TPR = D / 16;                 // threads per row, 8 pairs each
  constexpr int RPB = 256 / TPR;              // rows per block per pass
  const int c = threadIdx.x % TPR;
  double g[8];                                // revolutions per position of each pair
  rope_revs8<D>(8 * c, log2_base, g);
  for (I r = (I)blockIdx.x * RPB + threadIdx.x / TPR; r < rows; r += (I)gridDim.x * RPB) {
    const int n = (int)((r / (I)Hx) % (I)N);  // rows are (batch, token, head), token-major
    const double pos = (double)n * pos_scale;
    const T* xr = x + r * D;
    T* yr = y + r * D;
    const v8<T> a = *reinterpret_cast<const v8<T>*>(xr + 8 * c);
    const v8<T> b = *reinterpret_cast<const v8<T>*>(xr + D / 2 + 8 * c);
    v8<T> ya, yb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float sn, cs;
      if constexpr (sizeof(T) == 2) {
        rope_cs(pos, g[e], cs, sn);
      } else {
        const double u = pos * g[e];
        const float fr = (float)(u - rint(u));    // the angle in revolutions, in [-1/2, 1/2]
        sincosf(fr * 6.28318530717958647692f, &sn, &cs);
      }
      if (inverse) sn = -sn;
      float y0, y1;
      rope_turn((float)a[e], (float)b[e], cs, sn, y0, y1);
      ya[e] = (T)y0;
      yb[e] = (T)y1;
    }
    *reinterpret_cast<v8<T>*>(yr + 8 * c) = ya;
    *reinterpret_cast<v8<T>*>(yr + D / 2 + 8 * c) = yb;
  }
}

template <typename T, int D>
hipError_t launch_rope(const void* x, void* y, int B, int N, int Hx, double pos_scale, double base, int inverse,
                       hipStream_t stream) {
  const long long rows = (long long)B * N * Hx;
  constexpr int RPB = 256 / (D / 16);
  const long long blocks = (rows + RPB - 1) / RPB;
  const unsigned grid = (unsigned)(blocks < 16384 ? blocks : 16384);   // grid-stride beyond 16384 blocks
  if (rows + (long long)grid * RPB < (1ll << 32))
    hipLaunchKernelGGL((s2attn_rope_kernel<T, D, unsigned>), dim3(grid), dim3(256), 0, stream, (const T*)x, (T*)y,
                       (unsigned)rows, N, Hx, pos_scale, log2(base), inverse);
  else
    hipLaunchKernelGGL((s2attn_rope_kernel<T, D, long long>), dim3(grid), dim3(256), 0, stream, (const T*)x, (T*)y,
                       rows, N, Hx, pos_scale, log2(base), inverse);
  return hipGetLastError();
}

template hipError_t launch_rope<bf16, 64>(const void*, void*, int, int, int, double, double, int, hipStream_t);
template hipError_t launch_rope<bf16, 128>(const void*, void*, int, int, int, double, double, int, hipStream_t);
template hipError_t launch_rope<float, 64>(const void*, void*, int, int, int, double, double, int, hipStream_t);
template hipError_t launch_rope<float, 128>(const void*, void*, int, int, int, double, double, int, hipStream_t);

}  // namespace s2a
