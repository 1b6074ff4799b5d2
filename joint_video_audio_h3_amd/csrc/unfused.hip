// Unfused epilogues (H3_UNFUSED=1): the block forward's fused GEMM epilogues
// written as separate, plain elementwise kernels that read the GEMM's fp32
// output (acc + bias, stored by the EPI_STORE epilogue).  They exist to A/B the
// fused epilogues on the device: each follows the definition of its step
// directly, with no staging, tiling or reordering.
//   qkv:    per (row, head) RMSNorm of the q and k sections with their gains,
//           the rotary turn of every channel pair, the q pre-scale
//           log2(e)/sqrt(d), and the head-major scatter (v transposed)
//           (minimax-h3-mlx README, "Architecture": 3-D RoPE on q and k;
//           H3-metal digest, "Checkpoint layout and media pipeline": QK
//           normalisation before RoPE)
//   swiglu: a = silu(z[:, :F]) * z[:, F:]  (mlx-h3 README / H3-metal digest,
//           the SwiGLU MLP)
//   resid:  x += gate[tag] * y  (minimax-h3-mlx README, "AdaLN: measure, do
//           not reason": the gated residual of each branch)
#include "h3_device.h"
#include "launch.h"

namespace h3 {

// One wavefront per (row, head); lane l owns channels 2l and 2l + 1 (a rotary
// pair) of each section.  Rows n .. n_pad-1 are written as zeros.
__global__ __launch_bounds__(64) void unfused_qkv_kernel(UnfusedQkvArgs a) {
  const int row = blockIdx.x, head = blockIdx.y, l = threadIdx.x;
  const int d = a.head_dim, half = d / 2;
  const bool on = l < half;
  const size_t qo = ((size_t)head * a.n_pad + row) * d + 2 * l;   // q, k [H][n_pad][d]
  const size_t vo = (size_t)head * d * a.n_pad + row;              // vt [H][d][n_pad]
  if (row >= a.n) {
    if (on) {
      *reinterpret_cast<uint32_t*>(a.q + qo) = 0u;
      *reinterpret_cast<uint32_t*>(a.k + qo) = 0u;
      a.vt[vo + (size_t)(2 * l) * a.n_pad] = 0;
      a.vt[vo + (size_t)(2 * l + 1) * a.n_pad] = 0;
    }
    return;
  }
  const float* u = a.u + (size_t)row * 3 * a.heads * d + (size_t)head * 3 * d;
  const float c = on ? a.cs[(size_t)row * d + 2 * l] : 0.f;
  const float s = on ? a.cs[(size_t)row * d + 2 * l + 1] : 0.f;
#pragma unroll
  for (int kind = 0; kind < 2; ++kind) {
    const float u0 = on ? u[kind * d + 2 * l] : 0.f;
    const float u1 = on ? u[kind * d + 2 * l + 1] : 0.f;
    const float ms = wave_sum(u0 * u0 + u1 * u1) / (float)d;
    const float rn = 1.0f / sqrtf(ms + a.eps);
    const uint16_t* gam = kind == 0 ? a.gq : a.gk;
    const float g0 = (on && gam) ? bf2f(gam[2 * l]) : 1.f;
    const float g1 = (on && gam) ? bf2f(gam[2 * l + 1]) : 1.f;
    const float x0 = u0 * rn * g0, x1 = u1 * rn * g1;
    float o0 = x0 * c - x1 * s, o1 = x0 * s + x1 * c;
    if (kind == 0) {
      o0 *= a.q_scale;
      o1 *= a.q_scale;
    }
    if (on) *reinterpret_cast<uint32_t*>((kind == 0 ? a.q : a.k) + qo) = pack2bf(o0, o1);
  }
  if (on) {
    a.vt[vo + (size_t)(2 * l) * a.n_pad] = f2bf(u[2 * d + 2 * l]);
    a.vt[vo + (size_t)(2 * l + 1) * a.n_pad] = f2bf(u[2 * d + 2 * l + 1]);
  }
}

// One thread per output element: a[r][c] = silu(z[r][c]) * z[r][F + c].
__global__ __launch_bounds__(256) void unfused_swiglu_kernel(const float* __restrict__ z, int64_t n, int F,
                                                             uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n * F) return;
  const int64_t r = i / F;
  const int c = (int)(i % F);
  const float g = z[r * 2 * F + c], v = z[r * 2 * F + F + c];
  out[i] = f2bf(g / (1.0f + expf(-g)) * v);
}

// One thread per element: x[r][c] += gate[tag[r]][c] * y[r][c].
__global__ __launch_bounds__(256) void unfused_resid_kernel(const float* __restrict__ y, int64_t n, int D,
                                                            const uint16_t* __restrict__ gate,
                                                            const int32_t* __restrict__ tag, int tag_stride,
                                                            float* __restrict__ x) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n * D) return;
  const int64_t r = i / D;
  const int c = (int)(i % D);
  x[i] += bf2f(gate[(size_t)tag[r] * tag_stride + c]) * y[i];
}

hipError_t launch_unfused_qkv(const UnfusedQkvArgs& a, hipStream_t s) {
  if (a.head_dim > 128 || a.head_dim % 2 != 0) return hipErrorInvalidValue;
  unfused_qkv_kernel<<<dim3(a.n_pad, a.heads), 64, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_unfused_swiglu(const float* z, int64_t n, int F, uint16_t* out, hipStream_t s) {
  const int64_t total = n * F;
  unfused_swiglu_kernel<<<dim3((unsigned)((total + 255) / 256)), 256, 0, s>>>(z, n, F, out);
  return hipGetLastError();
}

hipError_t launch_unfused_resid(const float* y, int64_t n, int D, const uint16_t* gate, const int32_t* tag,
                                int tag_stride, float* x, hipStream_t s) {
  const int64_t total = n * D;
  unfused_resid_kernel<<<dim3((unsigned)((total + 255) / 256)), 256, 0, s>>>(y, n, D, gate, tag, tag_stride, x);
  return hipGetLastError();
}

}  // namespace h3
